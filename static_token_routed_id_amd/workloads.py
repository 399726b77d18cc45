"""Seeded synthetic inputs for the L3 layer (Large Lookup Layer).

This module only *draws* inputs. It holds none of the layer's arithmetic, so
both the CPU oracle (via the tests) and the HIP path (via the binding) can be
fed the same arrays without sharing any method code.

What the inputs stand for (gist.science explainer of "L^3: Large Lookup
Layers", Technical Summary):
  * Core Architecture: token id t selects a pre-computed subset of a large
    embedding table; K_t and V_t are the key / value rows of that subset.
  * Information-Theoretic Embedding Allocation: every token gets between 1 and
    k (e.g. 512) rows and the allocation is heavy-tailed. Here a capped,
    frequency-proportional count stands in for the paper's corpus-driven
    allocation, and Zipf-distributed ids stand in for natural-text tokens.

Recipe (draws in float64 -- tables in float32 -- then rounded once to the
storage dtype):
  * f_t = (t+1)^-s / sum_u (u+1)^-s over t in [0, V)  (id = frequency rank)
  * n_t = clamp(floor(budget * f_t), 1, cap); offsets = exclusive prefix sum
  * ids ~ Categorical(f) through the inverse CDF of uniform draws
  * K ~ N(0, sigma_k), V ~ N(0, sigma_v), W_up ~ N(0, 1/sqrt(d_e)),
    W_mix ~ N(0, 1/sqrt(2d)), gamma = 1, beta = 0, x ~ N(0, 1), dy ~ N(0, 1)
    (sigma is a standard deviation)
  * every stream has its own numpy PCG64 generator seeded with
    SeedSequence([0x4C33, config, stream, block]); tables are drawn in blocks
    of 65536 rows so they can be filled in parallel.

Storage: float32 configs keep float32 arrays; bf16 configs keep uint16 arrays
holding bfloat16 bit patterns (round-to-nearest-even of the float64 draw via
float32). ``decode`` turns either into float64 for the oracle.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

SEED_ROOT = 0x4C33
TABLE_BLOCK = 65536

# stream numbers of SeedSequence([SEED_ROOT, config, stream, block])
S_IDS, S_X, S_K, S_V, S_WUP, S_WMIX, S_DY, S_SHUFFLE, S_LNPARAM = range(9)


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and distribution of one synthetic workload."""
    name: str
    dtype: str            # "f32" or "bf16": storage / compute-input dtype
    vocab: int
    zipf_s: float         # exponent of the id / allocation Zipf law
    budget: int           # embedding budget spread over the vocabulary
    cap: int              # per-token row cap (the pages' k)
    d: int                # hidden width (= key width)
    d_e: int              # value width
    batch: int            # tokens per call
    sigma_k: float
    sigma_v: float
    hot_frac: float = 0.0     # fraction of tokens forced onto id 0
    hot_rows: int = 0         # rows given to the hot id (0 = no override)
    hot_id_zipf_s: float = 0.0  # Zipf exponent of the non-hot ids
    training: bool = False    # also draw an upstream gradient dy
    k_max: int = 512


SPECS = {
    # tiny fp32 forward
    "tiny_fp32": Spec("tiny_fp32", "f32", 256, 1.1, 2048, 32, 64, 64, 512,
                      1.0 / 8, 1.0 / 8),
    # prefill-shaped bf16 forward (4 x 2048 tokens flattened)
    "prefill_bf16": Spec("prefill_bf16", "bf16", 32768, 1.0, 1 << 18, 512,
                         1024, 256, 8192, 1.0 / 32, 1.0 / 16),
    # decode-shaped bf16 forward (64 tokens per step)
    "decode_bf16": Spec("decode_bf16", "bf16", 65536, 1.0, 1 << 20, 512,
                        2048, 512, 64, 1.0 / np.sqrt(2048), 1.0 / np.sqrt(512)),
    # large prefill bf16 forward
    "large_prefill_bf16": Spec("large_prefill_bf16", "bf16", 131072, 1.05,
                               1 << 22, 512, 2048, 512, 65536,
                               1.0 / np.sqrt(2048), 1.0 / np.sqrt(512)),
    # training step: tiny shapes, 30% of tokens on id 0 which has 512 rows
    "train_skew_bf16": Spec("train_skew_bf16", "bf16", 256, 1.1, 2048, 32,
                            64, 64, 512, 1.0 / 8, 1.0 / 8, hot_frac=0.3,
                            hot_rows=512, hot_id_zipf_s=1.0, training=True),
    # the same skew at the prefill shapes (d = 1024, d_e = 256, 8192 tokens,
    # 30% of them on id 0, which has 512 rows)
    "train_skew_prefill_bf16": Spec("train_skew_prefill_bf16", "bf16", 32768,
                                    1.0, 1 << 18, 512, 1024, 256, 8192,
                                    1.0 / 32, 1.0 / 16, hot_frac=0.3,
                                    hot_rows=512, hot_id_zipf_s=1.0,
                                    training=True),
}
# index order used by the measurement configs
CONFIG_ORDER = ["tiny_fp32", "prefill_bf16", "decode_bf16",
                "large_prefill_bf16", "train_skew_bf16",
                "train_skew_prefill_bf16"]


def _rng(cfg: int, stream: int, block: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([SEED_ROOT, cfg, stream, block])))


# ---------------------------------------------------------------- dtypes ---
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def store(a64: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float64 draw once into the storage dtype."""
    a32 = np.asarray(a64, dtype=np.float32)
    return a32 if dtype == "f32" else f32_to_bf16_bits(a32)


def decode(a: np.ndarray) -> np.ndarray:
    """Storage array (float32 or bf16 bits) -> float64 values."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


class Rows:
    """Row view of a stored table that decodes slices to float64 on access."""

    def __init__(self, table: np.ndarray):
        self.table = table
        self.shape = table.shape

    def __getitem__(self, idx):
        return decode(self.table[idx])

    def __len__(self):
        return self.table.shape[0]


# ------------------------------------------------------------ allocation ---
def zipf_freq(vocab: int, s: float) -> np.ndarray:
    r = np.arange(1, vocab + 1, dtype=np.float64)
    f = r ** (-s)
    return f / f.sum()


def allocation(spec: Spec) -> np.ndarray:
    """Rows per token id: clamp(floor(budget * f_t), 1, cap) (int64)."""
    f = zipf_freq(spec.vocab, spec.zipf_s)
    n = np.clip(np.floor(spec.budget * f), 1, spec.cap).astype(np.int64)
    if spec.hot_rows:
        n[0] = spec.hot_rows
    return n


def offsets_from_counts(n: np.ndarray) -> np.ndarray:
    off = np.zeros(n.shape[0] + 1, dtype=np.int64)
    np.cumsum(n, out=off[1:])
    return off


def draw_ids(rng: np.random.Generator, freq: np.ndarray, count: int,
             first: int = 0) -> np.ndarray:
    cdf = np.cumsum(freq)
    cdf /= cdf[-1]
    u = rng.random(count)
    ids = np.searchsorted(cdf, u, side="right")
    return (np.minimum(ids, freq.shape[0] - 1) + first).astype(np.int32)


def batch_ids(spec: Spec, cfg: int, batch: Optional[int] = None) -> np.ndarray:
    B = spec.batch if batch is None else batch
    rng = _rng(cfg, S_IDS)
    if spec.hot_frac <= 0:
        return draw_ids(rng, zipf_freq(spec.vocab, spec.zipf_s), B)
    hot = int(round(spec.hot_frac * B))
    # the Zipf law over all ids, restricted to ids 1..V-1 and renormalised
    rest_f = zipf_freq(spec.vocab, spec.hot_id_zipf_s)[1:]
    rest = draw_ids(rng, rest_f / rest_f.sum(), B - hot, first=1)
    ids = np.concatenate([np.zeros(hot, np.int32), rest])
    perm = _rng(cfg, S_SHUFFLE).permutation(B)
    return ids[perm].astype(np.int32)


# ---------------------------------------------------------------- tables ---
_SUB_ROWS_ELEMS = 1 << 20  # elements drawn per sub-chunk (4 MB of float32)


def _fill_block(out_block: np.ndarray, cfg: int, stream: int, block: int,
                sigma: float) -> None:
    """Fill one table block with N(0, sigma) draws (float32 generator).

    Tables are drawn in float32 (they end as bf16 or float32 anyway), in
    sub-chunks of whole rows through reused buffers, and rounded straight
    into the output; fresh multi-GB temporaries are never allocated.
    """
    g = _rng(cfg, stream, block)
    rows, cols = out_block.shape
    step = max(1, _SUB_ROWS_ELEMS // cols)
    buf = np.empty((step, cols), np.float32)
    tmp = np.empty((step, cols), np.uint32) if out_block.dtype == np.uint16 \
        else None
    sig = np.float32(sigma)
    for r0 in range(0, rows, step):
        n = min(step, rows - r0)
        b = buf[:n]
        g.standard_normal(out=b, dtype=np.float32)
        np.multiply(b, sig, out=b)
        if tmp is None:
            out_block[r0:r0 + n] = b
        else:
            u = b.view(np.uint32)
            t = tmp[:n]
            # round to nearest even: u + 0x7FFF + ((u >> 16) & 1), then >> 16
            np.right_shift(u, np.uint32(16), out=t)
            np.bitwise_and(t, np.uint32(1), out=t)
            np.add(t, np.uint32(0x7FFF), out=t)
            np.add(t, u, out=t)
            np.right_shift(t, np.uint32(16), out=t)
            np.copyto(out_block[r0:r0 + n], t, casting="unsafe")


def draw_table(cfg: int, stream: int, rows: int, cols: int, sigma: float,
               dtype: str, threads: Optional[int] = None) -> np.ndarray:
    """Table of rows x cols N(0, sigma) drawn in 65536-row blocks."""
    out = np.empty((rows, cols), np.float32 if dtype == "f32" else np.uint16)
    nblk = (rows + TABLE_BLOCK - 1) // TABLE_BLOCK

    def fill(b):
        r0 = b * TABLE_BLOCK
        r1 = min(rows, r0 + TABLE_BLOCK)
        _fill_block(out[r0:r1], cfg, stream, b, sigma)

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if nblk == 1 or threads <= 1:
        for b in range(nblk):
            fill(b)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nblk)))
    return out


@dataclasses.dataclass
class Workload:
    spec: Spec
    cfg: int
    ids: np.ndarray        # int32 [B]
    offsets: np.ndarray    # int64 [V+1]
    x: np.ndarray          # [B, d]
    K: np.ndarray          # [R, d]
    V: np.ndarray          # [R, d_e]
    W_up: np.ndarray       # [d, d_e]
    gamma: np.ndarray      # [d]
    beta: np.ndarray       # [d]
    W_mix: np.ndarray      # [d, 2d]
    dy: Optional[np.ndarray] = None  # [B, d]

    @property
    def rows(self) -> int:
        return int(self.offsets[-1])

    @property
    def batch(self) -> int:
        return int(self.ids.shape[0])


def make(name_or_index, batch: Optional[int] = None, ln_perturb: bool = False,
         threads: Optional[int] = None) -> Workload:
    """Draw the workload named (or indexed) ``name_or_index``.

    ``batch`` overrides the token count (ids are the first draws of the same
    stream); ``ln_perturb`` replaces gamma=1, beta=0 with gamma ~ 1+N(0,0.2),
    beta ~ N(0,0.2) so that tests exercise the affine part of LayerNorm.
    """
    if isinstance(name_or_index, int):
        cfg = name_or_index
        spec = SPECS[CONFIG_ORDER[cfg]]
    else:
        spec = SPECS[name_or_index]
        cfg = CONFIG_ORDER.index(spec.name)
    return make_from_spec(spec, cfg, batch, ln_perturb, threads)


def make_from_spec(spec: Spec, cfg: int, batch: Optional[int] = None,
                   ln_perturb: bool = False,
                   threads: Optional[int] = None) -> Workload:
    """Draw a workload of any Spec (e.g. the edge-case shapes of the tests)
    from the streams of configuration number cfg."""
    B = spec.batch if batch is None else batch
    counts = allocation(spec)
    offsets = offsets_from_counts(counts)
    R = int(offsets[-1])
    dt = spec.dtype
    ids = batch_ids(spec, cfg, B)
    x = store(_rng(cfg, S_X).standard_normal((B, spec.d)), dt)
    K = draw_table(cfg, S_K, R, spec.d, spec.sigma_k, dt, threads)
    V = draw_table(cfg, S_V, R, spec.d_e, spec.sigma_v, dt, threads)
    W_up = store(_rng(cfg, S_WUP).standard_normal((spec.d, spec.d_e))
                 / np.sqrt(spec.d_e), dt)
    W_mix = store(_rng(cfg, S_WMIX).standard_normal((spec.d, 2 * spec.d))
                  / np.sqrt(2 * spec.d), dt)
    if ln_perturb:
        g = _rng(cfg, S_LNPARAM)
        gamma = store(1.0 + 0.2 * g.standard_normal(spec.d), dt)
        beta = store(0.2 * g.standard_normal(spec.d), dt)
    else:
        gamma = store(np.ones(spec.d), dt)
        beta = store(np.zeros(spec.d), dt)
    dy = None
    if spec.training:
        dy = store(_rng(cfg, S_DY).standard_normal((B, spec.d)), dt)
    return Workload(spec, cfg, ids, offsets, x, K, V, W_up, gamma, beta,
                    W_mix, dy)


def upstream_grad(w: Workload) -> np.ndarray:
    """dy for a training step: the workload's own, else drawn from the same
    seeded stream a training workload of this configuration would use."""
    if w.dy is not None:
        return w.dy
    return store(_rng(w.cfg, S_DY).standard_normal((w.batch, w.spec.d)),
                 w.spec.dtype)


def layer_params(w: Workload, layer: int,
                 threads: Optional[int] = None) -> Workload:
    """Layer `layer` of a stack sharing this batch's ids and offsets: its own
    K, V, W_up, W_mix drawn from streams of their own (layer 0 is w itself);
    x, gamma, beta and dy are w's."""
    if layer == 0:
        return w
    spec, cfg, dt = w.spec, w.cfg, w.spec.dtype
    off = 16 * layer
    K = draw_table(cfg, S_K + off, w.rows, spec.d, spec.sigma_k, dt, threads)
    V = draw_table(cfg, S_V + off, w.rows, spec.d_e, spec.sigma_v, dt,
                   threads)
    W_up = store(_rng(cfg, S_WUP + off).standard_normal((spec.d, spec.d_e))
                 / np.sqrt(spec.d_e), dt)
    W_mix = store(_rng(cfg, S_WMIX + off).standard_normal((spec.d, 2 * spec.d))
                  / np.sqrt(2 * spec.d), dt)
    return dataclasses.replace(w, K=K, V=V, W_up=W_up, W_mix=W_mix)


def with_u_offset(w: Workload, ratio: float) -> Workload:
    """Same inputs, W_up + ratio * 1 w0^T with w0 ~ N(0, 1/d_e) from a stream
    of its own: every row of W_up gains the same vector, so each token's
    up-projection gains one common value (a . w0 * ratio) over all d
    columns, about `ratio` times the spread of its other entries. A LayerNorm
    input far from zero mean, for checking how the normalisation copes."""
    spec, dt = w.spec, w.spec.dtype
    w0 = _rng(w.cfg, S_WUP + 8).standard_normal(spec.d_e) / np.sqrt(spec.d_e)
    W_up = decode(w.W_up) + ratio * np.outer(np.ones(spec.d), w0)
    return dataclasses.replace(w, W_up=store(W_up, dt))


def with_ids(w: Workload, ids: np.ndarray, x: Optional[np.ndarray] = None,
             dy: Optional[np.ndarray] = None) -> Workload:
    """Same tables and weights, a different id stream (and optionally x, dy)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    B = ids.shape[0]
    dt = w.spec.dtype
    if x is None:
        x = store(_rng(w.cfg, S_X, 1 + B).standard_normal((B, w.spec.d)), dt)
    if dy is None and w.dy is not None:
        dy = store(_rng(w.cfg, S_DY, 1 + B).standard_normal((B, w.spec.d)), dt)
    return dataclasses.replace(w, ids=ids, x=x, dy=dy)


# ------------------------------------------------------------ corpora ---
# Seed config of the synthetic corpora (not one of the layer workloads).
CORPUS_CFG = 100


def synthetic_corpus(vocab: int, n_tokens: int, seed: int = 0,
                     zipf_s: float = 1.0, phrases: int = 0,
                     max_len: int = 6) -> np.ndarray:
    """A seeded token stream with the repetition structure of text, for the
    embedding allocation (the pages scan a natural-text corpus; none is
    here): a phrase book of `phrases` (default 8 * vocab) phrases of 1 to
    `max_len` tokens, their tokens drawn from Zipf(zipf_s) over the
    vocabulary, and the corpus a concatenation of phrases drawn from
    Zipf(zipf_s) over the book, cut to n_tokens (int32)."""
    P = phrases or 8 * vocab
    g = _rng(CORPUS_CFG, seed, 0)
    lens = g.integers(1, max_len + 1, P)
    starts = np.zeros(P + 1, np.int64)
    np.cumsum(lens, out=starts[1:])
    book = draw_ids(g, zipf_freq(vocab, zipf_s), int(starts[-1]))
    mean_len = float(lens.mean())
    picks = draw_ids(_rng(CORPUS_CFG, seed, 1), zipf_freq(P, zipf_s),
                     int(n_tokens / mean_len * 1.2) + 16)
    out = np.empty(0, np.int32)
    while out.shape[0] < n_tokens:
        seg = np.concatenate([book[starts[p]:starts[p + 1]] for p in picks])
        out = np.concatenate([out, seg])
    return np.ascontiguousarray(out[:n_tokens], dtype=np.int32)


def with_offsets(w: Workload, offsets: np.ndarray, ids: np.ndarray,
                 threads: Optional[int] = None) -> Workload:
    """Same shapes and weights, another allocation: tables of offsets[-1]
    rows drawn from this configuration's streams, the id stream `ids`, and x
    (and dy) drawn for that many tokens. The counts behind `offsets` are
    the caller's (e.g. an allocation scanned from a corpus)."""
    spec, cfg, dt = w.spec, w.cfg, w.spec.dtype
    offsets = np.ascontiguousarray(offsets, dtype=np.int64)
    R = int(offsets[-1])
    K = draw_table(cfg, S_K, R, spec.d, spec.sigma_k, dt, threads)
    V = draw_table(cfg, S_V, R, spec.d_e, spec.sigma_v, dt, threads)
    w2 = dataclasses.replace(w, offsets=offsets, K=K, V=V)
    return with_ids(w2, ids)


def decoded(w: Workload) -> dict:
    """float64 copies of every (small) array, for the oracle."""
    out = dict(ids=w.ids.astype(np.int64), offsets=w.offsets.copy(),
               x=decode(w.x), K=Rows(w.K), V=Rows(w.V), W_up=decode(w.W_up),
               gamma=decode(w.gamma), beta=decode(w.beta),
               W_mix=decode(w.W_mix))
    if w.dy is not None:
        out["dy"] = decode(w.dy)
    return out
