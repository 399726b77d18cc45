"""CPU oracle of the L3 (Large Lookup Layer) forward and backward pass.

TEST INFRASTRUCTURE ONLY. This module is the slow, obviously-correct
definition that the HIP library is checked against. Only the tests, the
smoke check and the benchmark's CPU-baseline leg may import it. It shares no
code with the HIP path and imports nothing from it.

Source of the method: gist.science explainer of "L^3: Large Lookup Layers"
(Tseng & De Sa, arXiv 2601.21461), Technical Summary:
  * Core Architecture / Mathematical Formulation: the layer outputs
        y = W_mix [ LayerNorm( W_up( V_t^T Softmax(K_t x) ) ) ; x ]
    where K_t, V_t are the embedding rows assigned to token id t.
  * Core Architecture / Static Routing: the rows are a pre-computed subset of
    a large table, selected by the token id alone.
  * Information-Theoretic Embedding Allocation / Constraints: every token
    owns between 1 and k rows (k = 512 in the pages' example).
  * Systems-Friendly Design / Batch Sorting: sorting a batch by token id makes
    the layer's attention mask block-diagonal (tokens of one id share K_t, V_t).

Readings where the pages are silent (each is a choice, listed here once):
  R1 key width = dim(x) = d; no query projection (the formula has none).
  R2 no 1/sqrt(d) temperature inside the softmax (the formula has none).
  R3 LayerNorm over the d features, biased variance, eps = 1e-5, affine
     gamma/beta; no bias in W_up or W_mix.
  R4 concat order [LayerNorm output ; x], so W_mix[:, :d] multiplies the
     LayerNorm output and W_mix[:, d:] multiplies x; weights are [out x in].
  R5 rows of id t are the contiguous slice offsets[t] : offsets[t+1].
  R6 the batch order is (id, original position); segments ascend by id.
  R7 an id outside [0, V) or a row count outside [1, k_max] is an error.
  R8 the backward pass is the chain rule of the forward (the pages print no
     gradients); table gradients are dense, untouched rows are zero.

Every floating-point step runs in float64 on the inputs as given (callers
pass the already-rounded fp32 / bf16 values decoded to float64).

Parity pins: every function here is pinned by the CPU tests (closed forms,
invariants, library routines, finite differences, brute force). Nothing here
is "parity unpinned".
"""
from __future__ import annotations

import itertools
from typing import Dict, Iterable, Optional

import numpy as np

LN_EPS = 1e-5


class OracleInputError(ValueError):
    """Raised for inputs the method does not define (reading R7)."""


# ------------------------------------------------------------------ plan ---
def plan(ids, offsets, vocab: int, k_max: int, rows: Optional[int] = None):
    """Sort the batch by token id and cut it into one segment per id.

    Systems-Friendly Design / Batch Sorting: after sorting by id, every token
    of one id reads the same K_t, V_t, so the mask is block-diagonal.
    The sort key is (id, original position), which is unique, so the
    permutation and the segments are unique (reading R6).

    Returns a dict with
      perm          int64 [B]   original token index at sorted position j
      S             int         number of distinct ids
      seg_id        int64 [S]   ascending ids
      seg_tok_start int64 [S+1] first sorted position of each segment, then B
      seg_row_off   int64 [S]   offsets[id]
      seg_n         int64 [S]   offsets[id+1] - offsets[id]
    """
    ids = [int(t) for t in np.asarray(ids).reshape(-1)]
    offsets = np.asarray(offsets, dtype=np.int64)
    if rows is None:
        rows = int(offsets[-1])
    for t in ids:
        if t < 0 or t >= vocab:
            raise OracleInputError(f"token id {t} outside [0, {vocab})")
    perm = sorted(range(len(ids)), key=lambda i: (ids[i], i))
    seg_id, seg_start, seg_off, seg_n = [], [], [], []
    pos = 0
    for t, grp in itertools.groupby(perm, key=lambda i: ids[i]):
        r0 = int(offsets[t])
        r1 = int(offsets[t + 1])
        n = r1 - r0
        if n < 1 or n > k_max or r0 < 0 or r1 > rows:
            raise OracleInputError(
                f"id {t} owns {n} rows [{r0}, {r1}); need 1..{k_max} inside "
                f"[0, {rows})")
        seg_id.append(t)
        seg_start.append(pos)
        seg_off.append(r0)
        seg_n.append(n)
        pos += len(list(grp))
    seg_start.append(pos)
    i64 = lambda v: np.asarray(v, dtype=np.int64)
    return dict(perm=i64(perm), S=len(seg_id), seg_id=i64(seg_id),
                seg_tok_start=i64(seg_start), seg_row_off=i64(seg_off),
                seg_n=i64(seg_n))


# ------------------------------------------------------- forward steps ---
# Core Architecture / Mathematical Formulation, one step per function.

def scores(Kt: np.ndarray, x: np.ndarray) -> np.ndarray:
    """s = K_t x (one score per row of the token's key slice)."""
    return Kt @ x


def softmax(s: np.ndarray) -> np.ndarray:
    """p = Softmax(s) over the token's rows (max-shifted, exact in fp64)."""
    e = np.exp(s - np.max(s))
    return e / np.sum(e)


def aggregate(Vt: np.ndarray, p: np.ndarray) -> np.ndarray:
    """a = V_t^T p."""
    return Vt.T @ p


def up(W_up: np.ndarray, a: np.ndarray) -> np.ndarray:
    """u = W_up a, W_up stored [d x d_e]; works row-wise on a batch a [.., d_e]."""
    return a @ W_up.T


def layernorm(u: np.ndarray, gamma, beta, eps: float = LN_EPS):
    """LayerNorm over the last axis (reading R3).

    Returns (h, uhat, mean, var) with uhat = (u - mean) / sqrt(var + eps).
    """
    mean = np.mean(u, axis=-1, keepdims=True)
    var = np.mean((u - mean) ** 2, axis=-1, keepdims=True)
    uhat = (u - mean) / np.sqrt(var + eps)
    return gamma * uhat + beta, uhat, mean[..., 0], var[..., 0]


def mix(W_mix: np.ndarray, h: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y = W_mix [h ; x], W_mix stored [d x 2d] (reading R4)."""
    return np.concatenate([h, x], axis=-1) @ W_mix.T


def _slice(offsets, t):
    r0 = int(offsets[t])
    return r0, int(offsets[t + 1]) - r0


def _tokens(B, tokens):
    return range(B) if tokens is None else [int(i) for i in tokens]


def aggregate_batch(x, ids, K, V, offsets, tokens: Optional[Iterable] = None):
    """a_i = V_t^T Softmax(K_t x_i) for each requested token, one at a time.

    K and V may be anything whose row slices convert to float64 arrays (a
    full table, or a view that decodes rows on demand).
    Returns (a [T, d_e], p list of per-token probability vectors).
    """
    toks = _tokens(len(ids), tokens)
    a_rows, p_rows = [], []
    for i in toks:
        r0, n = _slice(offsets, ids[i])
        Kt = np.asarray(K[r0:r0 + n], dtype=np.float64)
        Vt = np.asarray(V[r0:r0 + n], dtype=np.float64)
        p = softmax(scores(Kt, np.asarray(x[i], dtype=np.float64)))
        a_rows.append(aggregate(Vt, p))
        p_rows.append(p)
    d_e = np.asarray(V[0:1]).shape[1]
    a = np.array(a_rows, dtype=np.float64).reshape(len(a_rows), d_e)
    return a, p_rows


def forward(x, ids, K, V, offsets, W_up, gamma, beta, W_mix,
            eps: float = LN_EPS, tokens: Optional[Iterable] = None) -> Dict:
    """L3 layer forward for the requested tokens (all by default).

    Tokens never interact (Core Architecture: the layer maps one hidden state
    and one token id to one output), so a subset can be computed alone.
    Returns y and the intermediates a, u, mean, var, uhat, h ([T, ...]).
    """
    toks = list(_tokens(len(ids), tokens))
    x = np.asarray(x, dtype=np.float64)
    a, p = aggregate_batch(x, ids, K, V, offsets, toks)
    u = up(np.asarray(W_up, np.float64), a)
    h, uhat, mean, var = layernorm(u, np.asarray(gamma, np.float64),
                                   np.asarray(beta, np.float64), eps)
    y = mix(np.asarray(W_mix, np.float64), h, x[toks])
    return dict(y=y, a=a, p=p, u=u, mean=mean, var=var, uhat=uhat, h=h,
                tokens=np.asarray(toks, dtype=np.int64))


# ------------------------------------------------------------- backward ---
def layernorm_backward(dh, gamma, uhat, var, eps: float = LN_EPS):
    """du from dh through h = gamma * (u - mean) / sqrt(var + eps) + beta."""
    g = gamma * dh
    return (g - np.mean(g) - uhat * np.mean(g * uhat)) / np.sqrt(var + eps)


def softmax_backward(p, dp):
    """ds from dp through p = Softmax(s): ds = p * (dp - p . dp)."""
    return p * (dp - p @ dp)


def backward(x, ids, K, V, offsets, W_up, gamma, beta, W_mix, dy,
             eps: float = LN_EPS) -> Dict:
    """Gradients of sum(y * dy) for the whole batch (reading R8).

    Per token (chain rule through the forward steps, in reverse):
      dh   = W_a^T dy_i,  dx_b = W_b^T dy_i           (W_a = W_mix[:, :d])
      g    = gamma * dh
      du   = (g - mean(g) - uhat * mean(g * uhat)) / sqrt(var + eps)
      da   = W_up^T du
      dp   = V_t da,      ds = p * (dp - p . dp)
      dx_i = dx_b + K_t^T ds
    Summed over tokens:
      dW_mix += dy_i [h ; x_i]^T, dgamma += dh * uhat, dbeta += dh,
      dW_up += du a^T, dV[rows of t] += p da^T, dK[rows of t] += ds x_i^T
    """
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    W_up = np.asarray(W_up, np.float64)
    W_mix = np.asarray(W_mix, np.float64)
    gamma = np.asarray(gamma, np.float64)
    beta = np.asarray(beta, np.float64)
    B, d = x.shape
    R = int(offsets[-1])
    d_e = W_up.shape[1]
    W_a, W_b = W_mix[:, :d], W_mix[:, d:]

    dx = np.zeros((B, d))
    dK = np.zeros((R, d))
    dV = np.zeros((R, d_e))
    dW_up = np.zeros_like(W_up)
    dW_mix = np.zeros_like(W_mix)
    dgamma = np.zeros(d)
    dbeta = np.zeros(d)
    for i in range(B):
        t = int(ids[i])
        r0, n = _slice(offsets, t)
        Kt = np.asarray(K[r0:r0 + n], dtype=np.float64)
        Vt = np.asarray(V[r0:r0 + n], dtype=np.float64)
        # recompute the forward for token i
        p = softmax(scores(Kt, x[i]))
        a = aggregate(Vt, p)
        u = up(W_up, a)
        h, uhat, _, var = layernorm(u, gamma, beta, eps)
        # reverse
        dh = W_a.T @ dy[i]
        dxb = W_b.T @ dy[i]
        du = layernorm_backward(dh, gamma, uhat, var, eps)
        da = W_up.T @ du
        dp = Vt @ da
        ds = softmax_backward(p, dp)
        dx[i] = dxb + Kt.T @ ds
        dW_mix += np.outer(dy[i], np.concatenate([h, x[i]]))
        dgamma += dh * uhat
        dbeta += dh
        dW_up += np.outer(du, a)
        dV[r0:r0 + n] += np.outer(p, da)
        dK[r0:r0 + n] += np.outer(ds, x[i])
    return dict(dx=dx, dK=dK, dV=dV, dW_up=dW_up, dgamma=dgamma, dbeta=dbeta,
                dW_mix=dW_mix)
