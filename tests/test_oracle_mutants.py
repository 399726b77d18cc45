"""Plant plausible mistakes in the oracle (on the CPU only) and require that
the pin suite catches every one: a dropped term, a wrong sign, a wrong index
or a transposed operand anywhere in the oracle must fail some pin."""
import numpy as np
import pytest

from oracle import l3_oracle as o
from tests.oracle_pins import ALL_PINS

_orig = {name: getattr(o, name) for name in
         ("scores", "softmax", "aggregate", "up", "layernorm", "mix",
          "layernorm_backward", "softmax_backward", "plan")}


def _ln_ddof1(u, gamma, beta, eps=o.LN_EPS):
    mean = np.mean(u, axis=-1, keepdims=True)
    var = np.var(u, axis=-1, ddof=1, keepdims=True)
    uhat = (u - mean) / np.sqrt(var + eps)
    return gamma * uhat + beta, uhat, mean[..., 0], var[..., 0]


def _ln_eps_outside(u, gamma, beta, eps=o.LN_EPS):
    mean = np.mean(u, axis=-1, keepdims=True)
    var = np.mean((u - mean) ** 2, axis=-1, keepdims=True)
    uhat = (u - mean) / (np.sqrt(var) + eps)
    return gamma * uhat + beta, uhat, mean[..., 0], var[..., 0]


def _ln_no_beta(u, gamma, beta, eps=o.LN_EPS):
    h, uhat, m, v = _orig["layernorm"](u, gamma, beta, eps)
    return gamma * uhat, uhat, m, v


def _ln_no_center(u, gamma, beta, eps=o.LN_EPS):
    mean = np.mean(u, axis=-1, keepdims=True)
    var = np.mean((u - mean) ** 2, axis=-1, keepdims=True)
    uhat = u / np.sqrt(var + eps)
    return gamma * uhat + beta, uhat, mean[..., 0], var[..., 0]


def _plan_unstable(ids, offsets, vocab, k_max, rows=None):
    pl = _orig["plan"](ids, offsets, vocab, k_max, rows)
    perm = pl["perm"].copy()
    st = pl["seg_tok_start"]
    for s in range(pl["S"]):  # reverse ties: breaks the (id, position) key
        perm[st[s]:st[s + 1]] = perm[st[s]:st[s + 1]][::-1]
    return dict(pl, perm=perm)


def _plan_bad_n(ids, offsets, vocab, k_max, rows=None):
    pl = _orig["plan"](ids, offsets, vocab, k_max, rows)
    return dict(pl, seg_n=pl["seg_n"] + 1)


MUTANTS = {
    "scores_scaled_by_sqrt_d": ("scores",
                                lambda Kt, x: Kt @ x / np.sqrt(x.shape[0])),
    "scores_sign": ("scores", lambda Kt, x: -(Kt @ x)),
    "softmax_unnormalised": ("softmax", lambda s: np.exp(s - np.max(s))),
    "softmax_min_shift_no_norm": ("softmax", lambda s: np.exp(np.min(s) - s)),
    "aggregate_uniform": ("aggregate",
                          lambda Vt, p: Vt.T @ np.full_like(p, 1 / len(p))),
    "aggregate_first_row": ("aggregate", lambda Vt, p: Vt[0] * p.sum()),
    "up_transposed": ("up", lambda W, a: a @ W if W.shape[0] == W.shape[1]
                      else (a @ W.T) * 1.01),
    "ln_unbiased_var": ("layernorm", _ln_ddof1),
    "ln_eps_outside_sqrt": ("layernorm", _ln_eps_outside),
    "ln_no_beta": ("layernorm", _ln_no_beta),
    "ln_not_centered": ("layernorm", _ln_no_center),
    "mix_concat_swapped": ("mix", lambda W, h, x:
                           np.concatenate([x, h], axis=-1) @ W.T),
    "mix_drops_x": ("mix", lambda W, h, x: h @ W[:, :h.shape[-1]].T),
    "lnb_drops_mean_g": ("layernorm_backward",
                         lambda dh, gamma, uhat, var, eps=o.LN_EPS:
                         (gamma * dh - uhat * np.mean(gamma * dh * uhat))
                         / np.sqrt(var + eps)),
    "lnb_sign": ("layernorm_backward",
                 lambda dh, gamma, uhat, var, eps=o.LN_EPS:
                 (gamma * dh - np.mean(gamma * dh)
                  + uhat * np.mean(gamma * dh * uhat)) / np.sqrt(var + eps)),
    "lnb_no_gamma": ("layernorm_backward",
                     lambda dh, gamma, uhat, var, eps=o.LN_EPS:
                     _orig["layernorm_backward"](dh, np.ones_like(gamma),
                                                 uhat, var, eps)),
    "smb_drops_centering": ("softmax_backward", lambda p, dp: p * dp),
    "smb_sign": ("softmax_backward", lambda p, dp: p * (dp + p @ dp)),
    "plan_ties_reversed": ("plan", _plan_unstable),
    "plan_wrong_counts": ("plan", _plan_bad_n),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(o, attr, fn)
    failures = []
    for pin in ALL_PINS:
        try:
            pin(o)
        except Exception as e:  # noqa: BLE001 - any failure counts
            failures.append(f"{pin.__name__}: {type(e).__name__}")
    assert failures, f"mutant {name} passed every pin"
