"""ctypes binding of libl3 (include/l3.h), with the C entry points' names.

Argument marshalling only: tensors become device pointers, the stream is the
current torch stream, and a non-zero status raises L3Error. Every step of the
computation runs in the HIP library. If libl3.so is missing this module
raises at import: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import (POINTER, Structure, byref, c_char_p, c_double, c_float,
                    c_int, c_int32, c_int64, c_size_t, c_void_p)

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libl3.so")

L3_OK = 0
L3_ERR_NULL = -1
L3_ERR_SHAPE = -2
L3_ERR_DTYPE = -3
L3_ERR_WORKSPACE = -4
L3_ERR_HIP = -5
L3_ERR_TOKEN_RANGE = -6
L3_ERR_COUNT = -7
L3_ERR_STATE = -8
L3_F32 = 0
L3_BF16 = 1
L3_MAX_ROWS_PER_ID = 512


class L3Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {l3_status_str(status)} ({status})")


class l3_desc(Structure):
    _fields_ = [("vocab", c_int64), ("rows", c_int64), ("d", c_int32),
                ("d_k", c_int32), ("d_e", c_int32), ("k_max", c_int32),
                ("dtype", c_int32), ("y_dtype", c_int32), ("ln_eps", c_float)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run "
            "`python -m static_token_routed_id_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    sig = {
        "l3_status_str": (c_char_p, [c_int]),
        "l3_stage_name": (c_char_p, [c_int]),
        "l3_workspace_size": (c_int, [POINTER(l3_desc), c_int64,
                                      POINTER(c_size_t), POINTER(c_size_t),
                                      POINTER(c_size_t)]),
        "l3_plan": (c_int, [POINTER(l3_desc), P, c_int64, P, P, c_size_t, P,
                            POINTER(c_void_p)]),
        "l3_replan": (c_int, [P, P, c_int64, P, P]),
        "l3_forward": (c_int, [P, P, P, P, P, P, P, P, P, P, c_size_t, P,
                               c_size_t, P]),
        "l3_forward_noalloc": (c_int, [P, P, P, P, P, P, P, P, P, P]),
        "l3_allocate": (c_int, [c_int, P, c_int64, c_int64, c_int64, c_int32,
                                P, P]),
        "l3_backward": (c_int, [P, P, P, P, P, P, P, P, P, P, c_size_t, P, P,
                                P, P, P, P, P, P, c_size_t, P]),
        "l3_plan_check": (c_int, [P, P]),
        "l3_stage_rows": (c_int, [P, P, P, P, P, c_int64, P]),
        "l3_stage_rows_dma": (c_int, [P, P, P, P, P, c_int64, P]),
        "l3_plan_export": (c_int, [P, P, P, P, P, P, P, P]),
        "l3_plan_info": (c_int, [P, POINTER(c_int64), c_int, P]),
        "l3_plan_release": (None, [P]),
        "l3_plan_tokens": (c_int64, [P]),
        "l3_timing_enable": (c_int, [P, c_int]),
        "l3_timing_read": (c_int, [P, POINTER(c_double), POINTER(c_int64),
                                   c_int, POINTER(c_int)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("l3_workspace_size", "l3_plan", "l3_replan", "l3_forward",
            "l3_forward_noalloc", "l3_allocate",
            "l3_backward", "l3_plan_check", "l3_plan_export", "l3_plan_info",
            "l3_plan_release", "l3_plan_tokens", "l3_status_str",
            "l3_timing_enable", "l3_timing_read", "l3_stage_name",
            "l3_stage_rows", "l3_stage_rows_dma")


def lib():
    return _lib


def l3_status_str(status: int) -> str:
    return _lib.l3_status_str(int(status)).decode()


def l3_stage_name(stage: int):
    s = _lib.l3_stage_name(int(stage))
    return s.decode() if s else None


def _check(status: int, where: str) -> None:
    if status != L3_OK:
        raise L3Error(status, where)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t):
    if t is None or isinstance(t, int):
        return 0
    return t.numel() * t.element_size()


def _act_dtype(code: int):
    import torch
    return torch.bfloat16 if code == L3_BF16 else torch.float32


def _arg(t, name, dtype=None, shape=None, cols=None, host=False,
         optional=False):
    """Checks one tensor argument before its address crosses the ABI: a
    contiguous tensor on the GPU (host=True: in host memory) with the given
    dtype and shape (`cols`: 2-D with that many columns, any rows). Raw
    integer addresses pass unchecked (the caller vouches for them); None
    passes only where the entry point takes NULL."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name}: a tensor is required")
    if isinstance(t, int):
        return
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t)}")
    if host and t.is_cuda:
        raise ValueError(f"{name}: must be in host memory")
    if not host and not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected "
                         f"{tuple(shape)}")
    if cols is not None and (t.dim() != 2 or t.shape[1] != cols):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected "
                         f"(rows, {cols})")


def _check_params(desc, K, V, W_up, gamma, beta, W_mix):
    act = _act_dtype(desc.dtype)
    d, d_e = desc.d, desc.d_e
    _arg(K, "K", act, cols=d)
    _arg(V, "V", act, cols=d_e)
    _arg(W_up, "W_up", act, (d, d_e))
    _arg(gamma, "gamma", act, (d,))
    _arg(beta, "beta", act, (d,))
    _arg(W_mix, "W_mix", act, (d, 2 * d))


def make_desc(vocab, rows, d, d_e, k_max=512, dtype=L3_BF16, y_dtype=L3_F32,
              ln_eps=1e-5, d_k=None) -> l3_desc:
    return l3_desc(int(vocab), int(rows), int(d), int(d if d_k is None else d_k),
                   int(d_e), int(k_max), int(dtype), int(y_dtype),
                   float(ln_eps))


def l3_workspace_size(desc: l3_desc, max_tokens: int):
    p, s, c = c_size_t(), c_size_t(), c_size_t()
    _check(_lib.l3_workspace_size(byref(desc), int(max_tokens), byref(p),
                                  byref(s), byref(c)), "l3_workspace_size")
    return p.value, s.value, c.value


class Plan:
    """Owns an l3_plan_t handle (released on garbage collection)."""

    def __init__(self, handle: int, desc: l3_desc, plan_ws):
        self.handle = handle
        self.desc = desc
        self.plan_ws = plan_ws  # keep the workspace alive

    @property
    def tokens(self) -> int:
        return int(_lib.l3_plan_tokens(self.handle))

    def __del__(self):
        h = getattr(self, "handle", None)
        # at interpreter exit the module's globals may already be gone
        # (the process releases everything then anyway)
        if h and _lib is not None:
            _lib.l3_plan_release(h)
            self.handle = None


def _check_ids(desc, ids, offsets):
    import torch
    B = 0 if ids is None else ids.numel()
    if B:
        _arg(ids, "ids", torch.int32)
        _arg(offsets, "offsets", torch.int64, (desc.vocab + 1,))


def l3_plan(desc: l3_desc, ids, offsets, plan_ws, stream=None,
            check_status=True) -> Plan:
    out = c_void_p()
    _check_ids(desc, ids, offsets)
    _arg(plan_ws, "plan_ws", optional=True)
    B = 0 if ids is None else ids.numel()
    st = _lib.l3_plan(byref(desc), _ptr(ids), B, _ptr(offsets), _ptr(plan_ws),
                      _nbytes(plan_ws), _stream(stream), byref(out))
    if out.value is None:
        _check(st, "l3_plan")
    plan = Plan(out.value, desc, plan_ws)
    if check_status:
        _check(st, "l3_plan")
    return plan


def l3_replan(plan: Plan, ids, offsets, stream=None) -> None:
    _check_ids(plan.desc, ids, offsets)
    B = 0 if ids is None else ids.numel()
    _check(_lib.l3_replan(plan.handle, _ptr(ids), B, _ptr(offsets),
                          _stream(stream)), "l3_replan")


def l3_forward(plan: Plan, x, K, V, W_up, gamma, beta, W_mix, y, save,
               scratch, stream=None) -> None:
    B = plan.tokens
    if B > 0:
        desc = plan.desc
        _arg(x, "x", _act_dtype(desc.dtype), (B, desc.d))
        _check_params(desc, K, V, W_up, gamma, beta, W_mix)
        _arg(y, "y", _act_dtype(desc.y_dtype), (B, desc.d))
        _arg(save, "save", optional=True)
        _arg(scratch, "scratch")
    _check(_lib.l3_forward(plan.handle, _ptr(x), _ptr(K), _ptr(V), _ptr(W_up),
                           _ptr(gamma), _ptr(beta), _ptr(W_mix), _ptr(y),
                           _ptr(save), _nbytes(save), _ptr(scratch),
                           _nbytes(scratch), _stream(stream)), "l3_forward")


L3_NOALLOC_SCRATCH_BYTES = 64 << 20


def l3_forward_noalloc(plan: Plan, x, K, V, W_up, gamma, beta, W_mix, y,
                       stream=None) -> None:
    """Inference forward whose scratch is the library's static device array
    (no workspace argument, nothing allocated)."""
    B = plan.tokens
    if B > 0:
        desc = plan.desc
        _arg(x, "x", _act_dtype(desc.dtype), (B, desc.d))
        _check_params(desc, K, V, W_up, gamma, beta, W_mix)
        _arg(y, "y", _act_dtype(desc.y_dtype), (B, desc.d))
    _check(_lib.l3_forward_noalloc(plan.handle, _ptr(x), _ptr(K), _ptr(V),
                                   _ptr(W_up), _ptr(gamma), _ptr(beta),
                                   _ptr(W_mix), _ptr(y), _stream(stream)),
           "l3_forward_noalloc")


def l3_backward(plan: Plan, dy, x, K, V, W_up, gamma, beta, W_mix, save, dx,
                dK, dV, dW_up, dgamma, dbeta, dW_mix, scratch,
                stream=None) -> None:
    import torch
    desc = plan.desc
    B, d, d_e, R = plan.tokens, desc.d, desc.d_e, desc.rows
    f32 = torch.float32
    if B > 0:
        act = _act_dtype(desc.dtype)
        _arg(dy, "dy", act, (B, d))
        _arg(x, "x", act, (B, d))
        _check_params(desc, K, V, W_up, gamma, beta, W_mix)
        _arg(save, "save")
        _arg(dx, "dx", f32, (B, d))
        _arg(scratch, "scratch")
    _arg(dK, "dK", f32, (R, d))
    _arg(dV, "dV", f32, (R, d_e))
    _arg(dW_up, "dW_up", f32, (d, d_e))
    _arg(dgamma, "dgamma", f32, (d,))
    _arg(dbeta, "dbeta", f32, (d,))
    _arg(dW_mix, "dW_mix", f32, (d, 2 * d))
    _check(_lib.l3_backward(plan.handle, _ptr(dy), _ptr(x), _ptr(K), _ptr(V),
                            _ptr(W_up), _ptr(gamma), _ptr(beta), _ptr(W_mix),
                            _ptr(save), _nbytes(save), _ptr(dx), _ptr(dK),
                            _ptr(dV), _ptr(dW_up), _ptr(dgamma), _ptr(dbeta),
                            _ptr(dW_mix), _ptr(scratch), _nbytes(scratch),
                            _stream(stream)), "l3_backward")


def l3_stage_rows(plan: Plan, K_host, V_host, K_stage, V_stage,
                  stream=None, dma=False) -> None:
    """Copy the batch's rows of host-resident tables into K_stage / V_stage
    (device, capacity = K_stage's rows) and point the plan at them; with
    dma=True the DMA engines copy (the call waits for `stream`)."""
    if plan.tokens > 0:
        act = _act_dtype(plan.desc.dtype)
        _arg(K_host, "K_host", act, (plan.desc.rows, plan.desc.d), host=True)
        _arg(V_host, "V_host", act, (plan.desc.rows, plan.desc.d_e),
             host=True)
        _arg(K_stage, "K_stage", act, cols=plan.desc.d)
        _arg(V_stage, "V_stage", act, cols=plan.desc.d_e)
        if (not isinstance(K_stage, int) and not isinstance(V_stage, int)
                and V_stage.shape[0] < K_stage.shape[0]):
            raise ValueError("V_stage holds fewer rows than K_stage")
    rows = int(K_stage.shape[0]) if K_stage is not None else 0
    fn = _lib.l3_stage_rows_dma if dma else _lib.l3_stage_rows
    _check(fn(plan.handle, _ptr(K_host), _ptr(V_host), _ptr(K_stage),
              _ptr(V_stage), rows, _stream(stream)),
           "l3_stage_rows_dma" if dma else "l3_stage_rows")


L3_ALLOC_UNIFORM = 0
L3_ALLOC_LZW = 1


def l3_allocate(method: int, corpus, vocab: int, budget: int,
                k_max: int = L3_MAX_ROWS_PER_ID):
    """Rows per token id (int64 [vocab]) and the offsets (int64 [vocab+1])
    from the embedding allocation; corpus is a host int32 array (numpy)."""
    if corpus is None:
        corpus = np.zeros(0, np.int32)
    corpus = np.ascontiguousarray(corpus)
    if corpus.dtype != np.int32 or corpus.ndim != 1:
        raise TypeError("corpus: a 1-D int32 numpy array is required")
    counts = np.zeros(max(int(vocab), 1), np.int64)
    offsets = np.zeros(max(int(vocab), 1) + 1, np.int64)
    P = lambda a: a.ctypes.data_as(c_void_p)
    _check(_lib.l3_allocate(int(method), P(corpus), corpus.shape[0],
                            int(vocab), int(budget), int(k_max), P(counts),
                            P(offsets)), "l3_allocate")
    return counts, offsets


def l3_plan_check(plan: Plan, stream=None) -> int:
    """Returns the plan's device-side status (0, or L3_ERR_TOKEN_RANGE /
    L3_ERR_COUNT / L3_ERR_WORKSPACE); raises only on a HIP failure."""
    st = _lib.l3_plan_check(plan.handle, _stream(stream))
    if st == L3_ERR_HIP or st == L3_ERR_NULL:
        raise L3Error(st, "l3_plan_check")
    return st


def l3_plan_export(plan: Plan, stream=None) -> dict:
    B = plan.tokens
    perm = np.zeros(max(B, 1), np.int32)
    S = np.zeros(1, np.int32)
    seg_id = np.zeros(max(B, 1), np.int32)
    seg_tok_start = np.zeros(B + 1, np.int32)
    seg_row_off = np.zeros(max(B, 1), np.int64)
    seg_n = np.zeros(max(B, 1), np.int32)
    P = lambda a: a.ctypes.data_as(c_void_p)
    _check(_lib.l3_plan_export(plan.handle, P(perm), P(S), P(seg_id),
                               P(seg_tok_start), P(seg_row_off), P(seg_n),
                               _stream(stream)), "l3_plan_export")
    n = int(S[0])
    return dict(perm=perm[:B].copy(), S=n, seg_id=seg_id[:n].copy(),
                seg_tok_start=seg_tok_start[:n + 1].copy(),
                seg_row_off=seg_row_off[:n].copy(), seg_n=seg_n[:n].copy())


def l3_plan_info(plan: Plan, stream=None) -> dict:
    v = (c_int64 * 6)()
    _check(_lib.l3_plan_info(plan.handle, v, 6, _stream(stream)),
           "l3_plan_info")
    keys = ("B", "S", "wave_items", "group_items", "chunk_rows",
            "group_min_rows")
    return {k: int(v[i]) for i, k in enumerate(keys)}


def l3_timing_enable(plan: Plan, enable: bool = True) -> None:
    _check(_lib.l3_timing_enable(plan.handle, 1 if enable else 0),
           "l3_timing_enable")


def l3_timing_read(plan: Plan) -> dict:
    n = c_int()
    ms = (c_double * 32)()
    cnt = (c_int64 * 32)()
    _check(_lib.l3_timing_read(plan.handle, ms, cnt, 32, byref(n)),
           "l3_timing_read")
    return {l3_stage_name(i): (ms[i], int(cnt[i])) for i in range(n.value)}
