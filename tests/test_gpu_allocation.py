"""The allocation feeding the layer: offsets from the LZW-variant scan of a
seeded synthetic corpus (computed by the oracle's allocation, which
tests/test_allocation.py checks l3_allocate against bit for bit), a batch
that is a window of the same corpus (its ids in text order), and the layer's
forward (inference and training) and the plan at the prefill shapes against
the fp64 oracle on every token."""
import functools

import numpy as np
import pytest

from oracle import allocation as A
from static_token_routed_id_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=1)
def _lzw_workload():
    base = gu.workload("prefill_bf16")
    V, budget, k = base.spec.vocab, base.spec.budget, base.spec.k_max
    corpus = wl.synthetic_corpus(V, 4_000_000, seed=11)
    counts = A.lzw(corpus, V, budget, k)
    ids = corpus[1_000_000:1_000_000 + base.batch]
    return wl.with_offsets(base, A.offsets(counts), ids), counts


def test_lzw_allocation_shape():
    w, counts = _lzw_workload()
    print(f"LZW allocation: rows {w.rows}, max {counts.max()}, at cap "
          f"{int((counts == 512).sum())}, median {np.median(counts)}")
    assert counts.min() >= 1 and counts.max() <= 512
    assert w.rows == counts.sum() <= (1 << 18)
    L = gu.lib()
    got, off = L.l3_allocate(L.L3_ALLOC_LZW, wl.synthetic_corpus(
        w.spec.vocab, 4_000_000, seed=11), w.spec.vocab, w.spec.budget, 512)
    assert np.array_equal(got, counts)


@pytest.mark.parametrize("training", [False, True])
def test_lzw_allocated_forward(training):
    w, _ = _lzw_workload()
    res = gu.run(w, training=training, nan_fill=True)
    gu.check_forward(w, res, gu.oracle_forward_parallel(w))


def test_lzw_allocated_plan():
    from oracle import l3_oracle
    w, _ = _lzw_workload()
    res = gu.run(w)
    L = gu.lib()
    got = L.l3_plan_export(res["layer"].plan)
    want = l3_oracle.plan(w.ids, w.offsets, w.spec.vocab, w.spec.k_max)
    for k in ("perm", "seg_id", "seg_tok_start", "seg_row_off", "seg_n"):
        assert np.array_equal(got[k], want[k]), k
    assert got["S"] == want["S"]
