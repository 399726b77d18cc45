"""Pins of the CPU oracle: checks against facts that do not come from it.

Every check takes the oracle module ``o`` and raises AssertionError when the
oracle disagrees with the fact. The plain tests run them on the oracle; the
mutant tests plant mistakes in the oracle (on the CPU) and require that at
least one check fails for each.

Facts used (formula: gist.science explainer of "L^3: Large Lookup Layers",
Technical Summary, Core Architecture, Mathematical Formulation):
  * closed forms: one row gives p = 1 and a = that V row; identical keys or a
    zero hidden state give a uniform softmax, so a = mean of V_t; two rows
    give a logistic weight; LayerNorm of a 2-vector; W_mix = [0 | I] gives y
    = x; a hand-derived example (tests/golden/hand_example.json)
  * invariants: joint row permutation of K_t, V_t; token permutation; the
    LayerNorm output does not change when W_up is scaled (eps = 0)
  * library routines: torch.softmax, F.layer_norm, F.linear in float64 and
    torch.autograd for the backward
  * finite differences of the forward for every backward output
  * backward identities: softmax gradients sum to zero over a token's rows;
    an id's dV rows sum to its tokens' da (torch autograd of the tail)
  * plan: numpy's stable lexsort and unique give the same sort and segments
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------- tiny inputs ---
def tiny_case(seed=0, vocab=6, d=5, d_e=3, B=9, counts=(1, 3, 2, 4, 1, 2),
              sigma_k=0.7, perturb_ln=True):
    rng = np.random.default_rng(seed)
    counts = np.asarray(counts[:vocab], dtype=np.int64)
    offsets = np.zeros(vocab + 1, np.int64)
    np.cumsum(counts, out=offsets[1:])
    R = int(offsets[-1])
    ids = rng.integers(0, vocab, B)
    ids[:3] = [1, 1, 3]  # make sure some ids repeat
    return dict(
        x=rng.standard_normal((B, d)), ids=ids, offsets=offsets,
        K=rng.standard_normal((R, d)) * sigma_k,
        V=rng.standard_normal((R, d_e)),
        W_up=rng.standard_normal((d, d_e)),
        gamma=(1 + 0.3 * rng.standard_normal(d)) if perturb_ln else np.ones(d),
        beta=(0.3 * rng.standard_normal(d)) if perturb_ln else np.zeros(d),
        W_mix=rng.standard_normal((d, 2 * d)) / np.sqrt(2 * d),
        dy=rng.standard_normal((B, d)), vocab=vocab)


def fwd(o, c, **kw):
    return o.forward(c["x"], c["ids"], c["K"], c["V"], c["offsets"],
                     c["W_up"], c["gamma"], c["beta"], c["W_mix"], **kw)


def bwd(o, c, **kw):
    return o.backward(c["x"], c["ids"], c["K"], c["V"], c["offsets"],
                      c["W_up"], c["gamma"], c["beta"], c["W_mix"], c["dy"],
                      **kw)


def close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


# ------------------------------------------------------- closed forms ---
def pin_single_row(o):
    """n_t = 1: softmax of one score is exactly 1, so a is that V row."""
    c = tiny_case(1)
    r = fwd(o, c)
    for j, i in enumerate(r["tokens"]):
        t = c["ids"][i]
        if c["offsets"][t + 1] - c["offsets"][t] == 1:
            assert np.array_equal(r["p"][j], [1.0]), "p != [1] for n_t = 1"
            assert np.array_equal(r["a"][j], c["V"][c["offsets"][t]]), \
                "a != V row for n_t = 1"


def pin_uniform(o):
    """Identical keys, or x = 0, give p = 1/n_t and a = mean(V_t)."""
    c = tiny_case(2)
    K = c["K"].copy()
    for t in range(c["vocab"]):
        r0, r1 = c["offsets"][t], c["offsets"][t + 1]
        K[r0:r1] = K[r0]
    c2 = dict(c, K=K)
    r = fwd(o, c2)
    c3 = dict(c, x=np.zeros_like(c["x"]))
    r3 = fwd(o, c3)
    for j, i in enumerate(r["tokens"]):
        t = c["ids"][i]
        r0, r1 = c["offsets"][t], c["offsets"][t + 1]
        mean = c["V"][r0:r1].mean(axis=0)
        close(r["a"][j], mean, 1e-13, "identical keys -> mean of V_t")
        close(r3["a"][j], mean, 1e-13, "x = 0 -> mean of V_t")


def pin_two_rows_logistic(o):
    """Two rows: p_0 = 1 / (1 + exp(s_1 - s_0))."""
    rng = np.random.default_rng(3)
    d, d_e = 4, 3
    x = rng.standard_normal((1, d))
    K = rng.standard_normal((2, d)) * 2.0
    V = rng.standard_normal((2, d_e))
    s0, s1 = float(K[0] @ x[0]), float(K[1] @ x[0])
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))
    r = o.forward(x, np.array([0]), K, V, np.array([0, 2]),
                  rng.standard_normal((d, d_e)), np.ones(d), np.zeros(d),
                  rng.standard_normal((d, 2 * d)))
    close(r["p"][0], [p0, 1.0 - p0], 1e-15, "logistic weight")
    close(r["a"][0], p0 * V[0] + (1.0 - p0) * V[1], 1e-14, "two-row mix")


def pin_layernorm_two(o):
    """LayerNorm of (u1, u2): uhat = +-(u1-u2)/2 / sqrt(((u1-u2)/2)^2 + eps)."""
    u = np.array([[0.3, -1.1], [2.0, 2.5], [7.0, -7.0]])
    gamma = np.array([1.5, -0.5])
    beta = np.array([0.25, 0.75])
    eps = 1e-5
    h, uhat, mean, var = o.layernorm(u, gamma, beta, eps)
    half = (u[:, 0] - u[:, 1]) / 2
    q = half / np.sqrt(half ** 2 + eps)
    close(uhat, np.stack([q, -q], axis=1), 1e-15, "LN 2-vector uhat")
    close(mean, u.mean(axis=1), 1e-15, "LN mean")
    close(var, half ** 2, 1e-15, "LN biased variance")
    close(h, np.stack([gamma[0] * q + beta[0], -gamma[1] * q + beta[1]], 1),
          1e-15, "LN affine")


def pin_mix_blocks(o):
    """W_mix = [0 | I] gives y = x; W_mix = [I | 0] gives y = LayerNorm part."""
    c = tiny_case(4)
    d = c["x"].shape[1]
    r = fwd(o, dict(c, W_mix=np.hstack([np.zeros((d, d)), np.eye(d)])))
    close(r["y"], c["x"], 0.0, "W_mix = [0 | I] -> y = x")
    r = fwd(o, dict(c, W_mix=np.hstack([np.eye(d), np.zeros((d, d))])))
    close(r["y"], r["h"], 0.0, "W_mix = [I | 0] -> y = h")


def pin_hand_example(o):
    """Hand-derived values from the formula (tests/golden/hand_example.json)."""
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        g = json.load(f)
    ev = lambda s: float(eval(s, {"__builtins__": {}}, {"sqrt": math.sqrt}))
    A = lambda k: np.asarray(g[k], dtype=np.float64)
    r = o.forward(A("x"), np.asarray(g["ids"]), A("K"), A("V"),
                  np.asarray(g["offsets"]), A("W_up"), A("gamma"), A("beta"),
                  A("W_mix"))
    exp = g["expected"]
    close(r["p"][0], [ev(s) for s in exp["p0"]], 1e-15, "hand example p")
    close(r["a"], [[ev(s) for s in row] for row in exp["a"]], 1e-14,
          "hand example a")
    close(r["y"], [[ev(s) for s in row] for row in exp["y"]], 1e-14,
          "hand example y")
    pl = o.plan(np.asarray(g["ids"]), np.asarray(g["offsets"]), g["vocab"],
                g["k_max"])
    assert list(pl["seg_n"]) == [2, 1] and pl["S"] == 2


# ---------------------------------------------------------- invariants ---
def pin_row_permutation(o):
    """Permuting the rows of every K_t and V_t jointly leaves y unchanged."""
    c = tiny_case(5)
    rng = np.random.default_rng(55)
    K, V = c["K"].copy(), c["V"].copy()
    for t in range(c["vocab"]):
        r0, r1 = c["offsets"][t], c["offsets"][t + 1]
        q = r0 + rng.permutation(r1 - r0)
        K[r0:r1], V[r0:r1] = c["K"][q], c["V"][q]
    close(fwd(o, dict(c, K=K, V=V))["y"], fwd(o, c)["y"], 1e-13,
          "joint row permutation")


def pin_token_permutation(o):
    """Tokens are independent: permuting the batch permutes y's rows."""
    c = tiny_case(6)
    q = np.random.default_rng(66).permutation(len(c["ids"]))
    r = fwd(o, dict(c, x=c["x"][q], ids=c["ids"][q]))
    close(r["y"], fwd(o, c)["y"][q], 1e-13, "token permutation")
    sub = fwd(o, c, tokens=[4, 1])
    close(sub["y"], fwd(o, c)["y"][[4, 1]], 0.0, "token subset")


def pin_ln_scale(o):
    """With eps = 0, y(alpha * W_up) = y(W_up) for alpha > 0."""
    c = tiny_case(7)
    y1 = fwd(o, c, eps=0.0)["y"]
    y2 = fwd(o, dict(c, W_up=3.7 * c["W_up"]), eps=0.0)["y"]
    close(y1, y2, 1e-12, "LayerNorm scale invariance")


# ---------------------------------------------------- library routines ---
def torch_layer(c, requires_grad=False):
    """Independent float64 formulation with torch library routines."""
    import torch
    import torch.nn.functional as F
    T = lambda a: torch.tensor(np.asarray(a, np.float64), dtype=torch.float64,
                               requires_grad=requires_grad)
    x, K, V = T(c["x"]), T(c["K"]), T(c["V"])
    W_up, gamma, beta, W_mix = T(c["W_up"]), T(c["gamma"]), T(c["beta"]), \
        T(c["W_mix"])
    d = x.shape[1]
    a_rows = []
    for i, t in enumerate(c["ids"]):
        r0, r1 = int(c["offsets"][t]), int(c["offsets"][t + 1])
        p = torch.softmax(torch.mv(K[r0:r1], x[i]), dim=0)
        a_rows.append(torch.mv(V[r0:r1].t(), p))
    a = torch.stack(a_rows)
    h = F.layer_norm(F.linear(a, W_up), (d,), gamma, beta, eps=1e-5)
    y = F.linear(torch.cat([h, x], dim=1), W_mix)
    return y, dict(x=x, K=K, V=V, W_up=W_up, gamma=gamma, beta=beta,
                   W_mix=W_mix)


def pin_torch_forward(o):
    c = tiny_case(8)
    y, _ = torch_layer(c)
    close(fwd(o, c)["y"], y.detach().numpy(), 1e-12, "torch forward")


def pin_torch_backward(o):
    import torch
    c = tiny_case(9)
    y, leaves = torch_layer(c, requires_grad=True)
    (y * torch.tensor(c["dy"])).sum().backward()
    g = bwd(o, c)
    names = dict(x="dx", K="dK", V="dV", W_up="dW_up", gamma="dgamma",
                 beta="dbeta", W_mix="dW_mix")
    for leaf, gname in names.items():
        close(g[gname], leaves[leaf].grad.numpy(), 1e-11,
              f"torch autograd {gname}")


# -------------------------------------------------- finite differences ---
def pin_finite_differences(o):
    """Central differences of L = sum(y * dy) against every gradient."""
    c = tiny_case(10, B=6)
    g = bwd(o, c)
    names = dict(x="dx", K="dK", V="dV", W_up="dW_up", gamma="dgamma",
                 beta="dbeta", W_mix="dW_mix")
    rng = np.random.default_rng(100)
    step = 1e-6

    def loss(cc):
        return float(np.sum(fwd(o, cc)["y"] * cc["dy"]))

    for leaf, gname in names.items():
        base = np.asarray(c[leaf], np.float64)
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in base.shape)
            plus, minus = base.copy(), base.copy()
            plus[idx] += step
            minus[idx] -= step
            fd = (loss(dict(c, **{leaf: plus}))
                  - loss(dict(c, **{leaf: minus}))) / (2 * step)
            an = g[gname][idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), \
                f"finite difference {gname}{idx}: fd {fd} vs {an}"


def pin_backward_identities(o):
    """Softmax gradients sum to zero over a token's rows (so the dK rows of an
    id sum to zero); one-row ids get no dK and dx = W_b^T dy; dbeta = W_a^T
    sum(dy); the dV rows of an id sum to the sum of that id's da."""
    c = tiny_case(11)
    g = bwd(o, c)
    d = c["x"].shape[1]
    for t in range(c["vocab"]):
        r0, r1 = c["offsets"][t], c["offsets"][t + 1]
        close(g["dK"][r0:r1].sum(axis=0), np.zeros(d), 1e-12,
              "dK rows of an id sum to 0")
        if r1 - r0 == 1:
            close(g["dK"][r0], np.zeros(d), 0.0, "dK = 0 for n_t = 1")
    W_a, W_b = c["W_mix"][:, :d], c["W_mix"][:, d:]
    close(g["dbeta"], W_a.T @ c["dy"].sum(axis=0), 1e-12, "dbeta")
    for i, t in enumerate(c["ids"]):
        if c["offsets"][t + 1] - c["offsets"][t] == 1:
            close(g["dx"][i], W_b.T @ c["dy"][i], 1e-12, "dx for n_t = 1")
    untouched = np.setdiff1d(np.arange(c["vocab"]), c["ids"])
    for t in untouched:
        r0, r1 = c["offsets"][t], c["offsets"][t + 1]
        close(g["dK"][r0:r1], 0 * g["dK"][r0:r1], 0.0, "untouched dK rows")
        close(g["dV"][r0:r1], 0 * g["dV"][r0:r1], 0.0, "untouched dV rows")
    # dV_t = sum_i p_i da_i^T and each p_i sums to one, so the dV rows of an
    # id add up to the sum of its tokens' da; da from torch autograd through
    # the layer's tail (LayerNorm of the up-projection, then W_mix) alone
    da = torch_tail_grad(c)
    for t in np.unique(c["ids"]):
        r0, r1 = c["offsets"][t], c["offsets"][t + 1]
        close(g["dV"][r0:r1].sum(axis=0), da[c["ids"] == t].sum(axis=0),
              1e-12, "dV rows of an id sum to its tokens' da")


def torch_tail_grad(c):
    """d(sum(y * dy))/da for the aggregate a, with torch routines: a from
    torch.softmax and matrix-vector products, then y = W_mix [LayerNorm(
    W_up a) ; x] under autograd with a as the leaf."""
    import torch
    import torch.nn.functional as F
    T = lambda v: torch.tensor(np.asarray(v, np.float64), dtype=torch.float64)
    x, K, V = T(c["x"]), T(c["K"]), T(c["V"])
    rows = []
    for i, t in enumerate(c["ids"]):
        r0, r1 = int(c["offsets"][t]), int(c["offsets"][t + 1])
        p = torch.softmax(torch.mv(K[r0:r1], x[i]), dim=0)
        rows.append(torch.mv(V[r0:r1].t(), p))
    a = torch.stack(rows).requires_grad_(True)
    d = x.shape[1]
    h = F.layer_norm(F.linear(a, T(c["W_up"])), (d,), T(c["gamma"]),
                     T(c["beta"]), eps=1e-5)
    y = F.linear(torch.cat([h, x], dim=1), T(c["W_mix"]))
    (y * T(c["dy"])).sum().backward()
    return a.grad.numpy()


# ------------------------------------------------------------------ plan ---
def pin_plan_lexsort(o):
    """The plan equals numpy's stable lexsort + unique, bit for bit."""
    rng = np.random.default_rng(12)
    vocab = 50
    counts = rng.integers(1, 9, vocab)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    for B in (0, 1, 7, 300):
        ids = rng.integers(0, vocab, B)
        pl = o.plan(ids, offsets, vocab, 8)
        perm = np.lexsort((np.arange(B), ids))
        assert np.array_equal(pl["perm"], perm), "perm"
        u, first, cnt = np.unique(ids[perm], return_index=True,
                                  return_counts=True)
        assert pl["S"] == len(u)
        assert np.array_equal(pl["seg_id"], u)
        assert np.array_equal(pl["seg_tok_start"],
                              np.concatenate([first, [B]]))
        assert np.array_equal(pl["seg_row_off"], offsets[u])
        assert np.array_equal(pl["seg_n"], counts[u])


def pin_plan_errors(o):
    """Ids outside [0, V) and row counts outside [1, k_max] are errors."""
    offsets = np.array([0, 2, 2, 5], np.int64)  # id 1 owns no row
    for ids, k_max in (([0, 3], 8), ([-1], 8), ([1], 8), ([2, 0], 2)):
        try:
            o.plan(np.array(ids), offsets, 3, k_max)
        except o.OracleInputError:
            continue
        raise AssertionError(f"plan accepted ids={ids} k_max={k_max}")
    o.plan(np.array([2, 0]), offsets, 3, 3)


ALL_PINS = [pin_single_row, pin_uniform, pin_two_rows_logistic,
            pin_layernorm_two, pin_mix_blocks, pin_hand_example,
            pin_row_permutation, pin_token_permutation, pin_ln_scale,
            pin_torch_forward, pin_torch_backward, pin_finite_differences,
            pin_backward_identities, pin_plan_lexsort, pin_plan_errors]
