"""Shared helpers of the GPU parity tests (device upload, runs, metrics)."""
from __future__ import annotations

import functools

import numpy as np
import pytest

from static_token_routed_id_amd import workloads as wl


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch


def lib():
    torch_cuda()
    from static_token_routed_id_amd import _lib
    return _lib


def l3_dtype(w: wl.Workload) -> int:
    from static_token_routed_id_amd import _lib
    return _lib.L3_BF16 if w.spec.dtype == "bf16" else _lib.L3_F32


def desc_of(w: wl.Workload, y_dtype=None, ln_eps=1e-5):
    from static_token_routed_id_amd import _lib
    return _lib.make_desc(w.spec.vocab, w.rows, w.spec.d, w.spec.d_e,
                          w.spec.k_max, l3_dtype(w),
                          _lib.L3_F32 if y_dtype is None else y_dtype, ln_eps)


class Dev:
    """Device copies of a workload's arrays."""

    def __init__(self, w: wl.Workload):
        from static_token_routed_id_amd.layer import to_device
        torch = torch_cuda()
        self.w = w
        self.ids = torch.from_numpy(w.ids).cuda()
        self.offsets = torch.from_numpy(w.offsets).cuda()
        for f in ("x", "K", "V", "W_up", "gamma", "beta", "W_mix"):
            setattr(self, f, to_device(getattr(w, f)))
        self.dy = to_device(w.dy) if w.dy is not None else None

    def params(self):
        return (self.x, self.K, self.V, self.W_up, self.gamma, self.beta,
                self.W_mix)


@functools.lru_cache(maxsize=4)
def workload(name, ln_perturb=False):
    return wl.make(name, ln_perturb=ln_perturb)


def run(w: wl.Workload, dev: Dev = None, training=False, y_dtype=None):
    """Plan + forward (+ backward when training). Returns a dict."""
    from static_token_routed_id_amd.layer import L3Layer
    torch = torch_cuda()
    dev = dev or Dev(w)
    layer = L3Layer(desc_of(w, y_dtype), w.batch, training=training)
    layer.make_plan(dev.ids, dev.offsets)
    y = layer.forward(*dev.params())
    out = dict(layer=layer, dev=dev, y=y)
    if training:
        B, d_e = w.batch, w.spec.d_e
        a32 = layer.save[: B * d_e * 4].view(torch.float32).view(B, d_e)
        out["a32"] = a32.clone()
    if training and dev.dy is not None:
        out["grads"] = layer.backward(dev.dy, *dev.params())
    torch.cuda.synchronize()
    return out


def oracle_forward(w: wl.Workload, tokens=None):
    from oracle import l3_oracle
    dd = wl.decoded(w)
    return l3_oracle.forward(dd["x"], dd["ids"], dd["K"], dd["V"],
                             dd["offsets"], dd["W_up"], dd["gamma"],
                             dd["beta"], dd["W_mix"], tokens=tokens)


def oracle_backward(w: wl.Workload):
    from oracle import l3_oracle
    dd = wl.decoded(w)
    return l3_oracle.backward(dd["x"], dd["ids"], dd["K"], dd["V"],
                              dd["offsets"], dd["W_up"], dd["gamma"],
                              dd["beta"], dd["W_mix"], dd["dy"])


def oracle_backward_sampled(w: wl.Workload, tokens, sample_ids):
    """Reference gradients of a whole training batch, sampled: dx rows of
    `tokens`, dK / dV rows of the ids in `sample_ids` (dict id -> [n, .]),
    and the weight gradients dW_mix, dW_up, dgamma, dbeta over every token.

    The oracle's own per-token steps (scores, softmax, aggregate, up,
    layernorm, layernorm_backward, softmax_backward) in the order of its
    backward; the weight gradients' sums over tokens are taken as one matrix
    product each (dy^T [H ; X], dU^T A) instead of per-token outer products,
    and the softmax backward runs only for the tokens the samples need.
    tests/test_oracle_sampled.py checks it against the oracle's backward."""
    from oracle import l3_oracle as O
    dd = wl.decoded(w)
    x, dy, ids, offsets = dd["x"], dd["dy"], dd["ids"], dd["offsets"]
    W_up, W_mix = dd["W_up"], dd["W_mix"]
    gamma, beta = dd["gamma"], dd["beta"]
    B, d = x.shape
    d_e = W_up.shape[1]
    W_a, W_b = W_mix[:, :d], W_mix[:, d:]
    tok_set = {int(t) for t in tokens}
    id_set = {int(t) for t in sample_ids}
    DH = dy @ W_a  # row i: W_a^T dy_i
    H = np.zeros((B, d))
    A = np.zeros((B, d_e))
    DU = np.zeros((B, d))
    UH = np.zeros((B, d))
    dx = {}
    dK = {}
    dV = {}
    for t in id_set:
        n = int(offsets[t + 1] - offsets[t])
        dK[t] = np.zeros((n, d))
        dV[t] = np.zeros((n, d_e))
    for i in range(B):
        t = int(ids[i])
        r0, r1 = int(offsets[t]), int(offsets[t + 1])
        Kt = np.asarray(dd["K"][r0:r1], dtype=np.float64)
        Vt = np.asarray(dd["V"][r0:r1], dtype=np.float64)
        p = O.softmax(O.scores(Kt, x[i]))
        a = O.aggregate(Vt, p)
        u = O.up(W_up, a)
        h, uhat, _, var = O.layernorm(u, gamma, beta)
        du = O.layernorm_backward(DH[i], gamma, uhat, var)
        H[i], A[i], DU[i], UH[i] = h, a, du, uhat
        if i in tok_set or t in id_set:
            da = W_up.T @ du
            ds = O.softmax_backward(p, Vt @ da)
            if i in tok_set:
                dx[i] = W_b.T @ dy[i] + Kt.T @ ds
            if t in id_set:
                dK[t] += np.outer(ds, x[i])
                dV[t] += np.outer(p, da)
    return dict(dx=dx, dK=dK, dV=dV,
                dW_mix=dy.T @ np.concatenate([H, x], axis=1),
                dW_up=DU.T @ A, dgamma=(DH * UH).sum(axis=0),
                dbeta=DH.sum(axis=0))


def f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_abs(g, o) -> float:
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    return float(np.max(np.abs(g - o))) if g.size else 0.0


def linf_rel(g, o) -> float:
    """max |g - o| / max |o| (the per-tensor relative error)."""
    o = np.asarray(o, np.float64)
    den = float(np.max(np.abs(o))) if o.size else 1.0
    return max_abs(g, o) / (den if den > 0 else 1.0)
