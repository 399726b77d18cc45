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


def aggregate_from_scratch(w: wl.Workload, scratch):
    """The aggregate a [B x d_e] in the activation dtype, which the forward
    leaves at the start of its scratch workspace (the W_up operand)."""
    torch = torch_cuda()
    B, d_e = w.batch, w.spec.d_e
    dt = torch.bfloat16 if w.spec.dtype == "bf16" else torch.float32
    es = 2 if w.spec.dtype == "bf16" else 4
    return scratch[: B * d_e * es].view(dt).view(B, d_e)


def run(w: wl.Workload, dev: Dev = None, training=False, y_dtype=None,
        nan_fill=False):
    """Plan + forward (+ backward when training). Returns a dict with y,
    the aggregate (float32 saved copy `a32` when training, the activation
    copy from scratch `a_act` otherwise) and the gradients.

    nan_fill: y, the save and scratch workspaces and every gradient start
    as NaN bit patterns, so a row or element that no kernel writes shows."""
    from static_token_routed_id_amd.layer import L3Layer, torch_dtype
    torch = torch_cuda()
    dev = dev or Dev(w)
    desc = desc_of(w, y_dtype)
    layer = L3Layer(desc, w.batch, training=training)
    y = None
    if nan_fill:
        layer.scratch.fill_(0xFF)
        if layer.save is not None:
            layer.save.fill_(0xFF)
        y = torch.full((w.batch, w.spec.d), float("nan"),
                       dtype=torch_dtype(desc.y_dtype), device="cuda")
    layer.make_plan(dev.ids, dev.offsets)
    y = layer.forward(*dev.params(), y=y)
    out = dict(layer=layer, dev=dev, y=y)
    B, d_e = w.batch, w.spec.d_e
    if training:
        a32 = layer.save[: B * d_e * 4].view(torch.float32).view(B, d_e)
        out["a32"] = a32.clone()
    else:
        out["a_act"] = aggregate_from_scratch(w, layer.scratch).clone()
    if training and dev.dy is not None:
        grads_out = None
        if nan_fill:
            d, R = w.spec.d, w.rows
            f32 = dict(dtype=torch.float32, device="cuda")
            nan = float("nan")
            grads_out = dict(dx=torch.full((B, d), nan, **f32),
                             dK=torch.full((R, d), nan, **f32),
                             dV=torch.full((R, d_e), nan, **f32),
                             dW_up=torch.full((d, d_e), nan, **f32),
                             dgamma=torch.full((d,), nan, **f32),
                             dbeta=torch.full((d,), nan, **f32),
                             dW_mix=torch.full((d, 2 * d), nan, **f32))
        out["grads"] = layer.backward(dev.dy, *dev.params(), out=grads_out)
    torch.cuda.synchronize()
    return out


F32_REL = 1e-4      # float32 workloads: max|g - o| / max|o| per tensor
BF16_ABS = 2e-2     # bf16 workloads: elementwise max|g - o| on y
A_BF16_ABS = 2e-3   # the aggregate itself on bf16 workloads (|a| < 0.5)


def check_forward(w: wl.Workload, res: dict, ref: dict, tokens=None):
    """y and the aggregate against the oracle's on the same tokens (all, or
    the rows `tokens` of the batch, in the order ref holds them). The
    aggregate is the float32 saved copy when training, else the activation
    copy (bf16 on bf16 workloads: its rounding, at most 2^-9 |a|, is inside
    the bound)."""
    y = f64(res["y"])
    a = f64(res["a32"]) if "a32" in res else (
        f64(res["a_act"]) if "a_act" in res else None)
    if tokens is not None:
        y = y[tokens]
        a = a[tokens] if a is not None else None
    assert np.isfinite(y).all(), "non-finite y"
    if a is not None:
        assert np.isfinite(a).all(), "non-finite aggregate"
    if w.spec.dtype == "f32":
        ey = linf_rel(y, ref["y"])
        print(f"{w.spec.name}: y linf-rel {ey:.3e}")
        assert ey <= F32_REL
        if a is not None:
            ea = linf_rel(a, ref["a"])
            print(f"{w.spec.name}: a linf-rel {ea:.3e}")
            assert ea <= F32_REL
    else:
        ey = max_abs(y, ref["y"])
        print(f"{w.spec.name}: y max abs {ey:.3e} (max|y| "
              f"{np.abs(ref['y']).max():.2f})")
        assert ey <= BF16_ABS
        if a is not None:
            ea = max_abs(a, ref["a"])
            print(f"{w.spec.name}: a max abs {ea:.3e}")
            assert ea <= A_BF16_ABS
    return dict(y=ey, a=ea if a is not None else None)


def oracle_forward(w: wl.Workload, tokens=None):
    from oracle import l3_oracle
    dd = wl.decoded(w)
    return l3_oracle.forward(dd["x"], dd["ids"], dd["K"], dd["V"],
                             dd["offsets"], dd["W_up"], dd["gamma"],
                             dd["beta"], dd["W_mix"], tokens=tokens)


class _LastSlice:
    """Row view of a stored table that keeps the last decoded slice: the
    oracle asks for one id's rows per token, and tokens taken in id order
    then decode each id once. Test plumbing only (no arithmetic)."""

    def __init__(self, table: np.ndarray):
        self.table = table
        self.shape = table.shape
        self.key = None
        self.val = None

    def __getitem__(self, idx):
        key = (idx.start, idx.stop) if isinstance(idx, slice) else None
        if key is not None and key == self.key:
            return self.val
        val = wl.decode(self.table[idx])
        if key is not None:
            self.key, self.val = key, val
        return val

    def __len__(self):
        return self.table.shape[0]


def oracle_forward_parallel(w: wl.Workload, tokens=None, threads=16,
                            chunk=1024):
    """oracle.forward over the requested tokens (default: all), in chunks of
    tokens taken in id order on a thread pool (numpy releases the GIL in its
    array work); BLAS single-threaded inside each worker. Returns y and a
    ([T, ...] in the order of `tokens`) and the token order."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import l3_oracle
    toks = np.arange(w.batch) if tokens is None else np.asarray(tokens)
    order = np.argsort(w.ids[toks], kind="stable")
    chunks = [toks[order[i:i + chunk]] for i in range(0, len(toks), chunk)]
    x = wl.decode(w.x)
    ids = w.ids.astype(np.int64)
    W_up, gamma, beta, W_mix = (wl.decode(w.W_up), wl.decode(w.gamma),
                                wl.decode(w.beta), wl.decode(w.W_mix))

    done = [0]

    def one(c):
        r = l3_oracle.forward(x, ids, _LastSlice(w.K), _LastSlice(w.V),
                              w.offsets, W_up, gamma, beta, W_mix, tokens=c)
        done[0] += 1
        if done[0] % 8 == 0:
            print(f"  oracle: {done[0]} of {len(chunks)} chunks", flush=True)
        return r["y"], r["a"]

    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(threads) as ex:
            parts = list(ex.map(one, chunks))
    pos = np.empty(len(toks), np.int64)
    pos[order] = np.arange(len(toks))
    y = np.concatenate([p[0] for p in parts])[pos]
    a = np.concatenate([p[1] for p in parts])[pos]
    return dict(y=y, a=a, tokens=toks)


def oracle_backward(w: wl.Workload):
    from oracle import l3_oracle
    dd = wl.decoded(w)
    return l3_oracle.backward(dd["x"], dd["ids"], dd["K"], dd["V"],
                              dd["offsets"], dd["W_up"], dd["gamma"],
                              dd["beta"], dd["W_mix"], dd["dy"])


def oracle_backward_sampled(w: wl.Workload, tokens, sample_ids, threads=16,
                            chunk=1024):
    """Reference gradients of a whole training batch, sampled: dx rows of
    `tokens`, dK / dV rows of the ids in `sample_ids` (dict id -> [n, .]),
    and the weight gradients dW_mix, dW_up, dgamma, dbeta over every token.

    The oracle's own per-token steps (scores, softmax, aggregate, up,
    layernorm, layernorm_backward, softmax_backward) in the order of its
    backward; the weight gradients' sums over tokens are taken as one matrix
    product each (dy^T [H ; X], dU^T A) instead of per-token outer products,
    and the softmax backward runs only for the tokens the samples need.
    Tokens run in id-ordered chunks on a thread pool (BLAS single-threaded
    inside each worker); an id's dK / dV adds its chunks' sums in chunk
    order. tests/test_oracle_sampled.py checks it against the oracle's
    backward."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import l3_oracle as O
    x, dy = wl.decode(w.x), wl.decode(w.dy)
    ids, offsets = w.ids.astype(np.int64), w.offsets
    W_up, W_mix = wl.decode(w.W_up), wl.decode(w.W_mix)
    gamma, beta = wl.decode(w.gamma), wl.decode(w.beta)
    B, d = x.shape
    d_e = W_up.shape[1]
    W_a, W_b = W_mix[:, :d], W_mix[:, d:]
    tok_set = {int(t) for t in tokens}
    id_set = {int(t) for t in sample_ids}
    H = np.zeros((B, d))
    A = np.zeros((B, d_e))
    DU = np.zeros((B, d))
    UH = np.zeros((B, d))
    order = np.argsort(ids, kind="stable")
    chunks = [order[i:i + chunk] for i in range(0, B, chunk)]

    def one(c):
        Kr, Vr = _LastSlice(w.K), _LastSlice(w.V)
        dx, dK, dV = {}, {}, {}
        c = [int(i) for i in c]
        P, Ac = [], np.zeros((len(c), d_e))
        for j, i in enumerate(c):
            t = int(ids[i])
            r0, r1 = int(offsets[t]), int(offsets[t + 1])
            p = O.softmax(O.scores(Kr[r0:r1], x[i]))
            Ac[j] = O.aggregate(Vr[r0:r1], p)
            P.append(p)
        # up-projection and LayerNorm row-wise over the chunk's tokens
        Uc = O.up(W_up, Ac)
        Hc, UHc, _, varc = O.layernorm(Uc, gamma, beta)
        DHc = dy[c] @ W_a
        for j, i in enumerate(c):
            t = int(ids[i])
            du = O.layernorm_backward(DHc[j], gamma, UHc[j], varc[j])
            H[i], A[i], DU[i], UH[i] = Hc[j], Ac[j], du, UHc[j]
            if i in tok_set or t in id_set:
                r0, r1 = int(offsets[t]), int(offsets[t + 1])
                Kt, Vt = Kr[r0:r1], Vr[r0:r1]
                p = P[j]
                da = W_up.T @ du
                ds = O.softmax_backward(p, Vt @ da)
                if i in tok_set:
                    dx[i] = W_b.T @ dy[i] + Kt.T @ ds
                if t in id_set:
                    if t not in dK:
                        dK[t] = np.zeros((r1 - r0, d))
                        dV[t] = np.zeros((r1 - r0, d_e))
                    dK[t] += np.outer(ds, x[i])
                    dV[t] += np.outer(p, da)
        return dx, dK, dV

    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(threads) as ex:
            parts = list(ex.map(one, chunks))
    dx, dK, dV = {}, {}, {}
    for t in id_set:
        n = int(offsets[t + 1] - offsets[t])
        dK[t] = np.zeros((n, d))
        dV[t] = np.zeros((n, d_e))
    for pdx, pdK, pdV in parts:
        dx.update(pdx)
        for t in pdK:
            dK[t] += pdK[t]
            dV[t] += pdV[t]
    DH = dy @ W_a
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
