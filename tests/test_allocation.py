"""The embedding allocation (CPU: the allocator is host code of libl3).

1. The oracle against its pins (tests/allocation_pins.py), and planted
   mistakes in the oracle each failing some pin.
2. l3_allocate against the oracle, bit for bit, on seeded synthetic corpora
   (caps reached and not, budgets reached and not), the uniform split, the
   offsets, and the error codes.

Parity of the allocation against the pages is unpinned: the pages give no
steps of their LZW variant and print no allocation (the oracle's header
lists the reading)."""
import numpy as np
import pytest

from oracle import allocation as A
from static_token_routed_id_amd import workloads as wl
from tests.allocation_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(A)


# ------------------------------------------------------------- mutants ---
_orig_parse = A.lzw_parse


def _mut_parse(kind):
    def parse(corpus, vocab, budget, k_max):
        toks = [int(t) for t in np.asarray(corpus).reshape(-1)]
        A._check(vocab, budget, k_max)
        for t in toks:
            if t < 0 or t >= vocab:
                raise A.AllocationInputError("token")
        counts = [1] * vocab
        dic = {(t,) for t in range(vocab)}
        entries, out = [], []
        total = vocab
        if not toks:
            return np.asarray(counts, np.int64), entries, out
        w = (toks[0],)
        for c in toks[1:]:
            if total >= budget + (1 if kind == "budget_off_by_one" else 0):
                break
            wc = w + (c,)
            if wc in dic and kind != "no_lookup":
                w = wc
                continue
            out.append(w)
            owner = wc[0] if kind == "first_token_owner" else c
            cap_ok = (counts[owner] <= k_max if kind == "cap_inclusive"
                      else counts[owner] < k_max)
            if cap_ok:
                dic.add(wc)
                entries.append(wc)
                counts[owner] += 1
                total += 1
            # LZ78's restart (the next phrase begins after c) instead of
            # LZW's (it begins at c)
            w = () if kind == "lz78_restart" else (c,)
        out.append(w)
        return np.asarray(counts, np.int64), entries, out
    return parse


def _mut_uniform_high(vocab, budget, k_max):
    A._check(vocab, budget, k_max)
    q, r = divmod(budget, vocab)
    return np.asarray([q + (1 if t >= vocab - r else 0) for t in range(vocab)],
                      np.int64)


MUTANTS = {
    "first_token_owner": ("lzw_parse", _mut_parse("first_token_owner")),
    "cap_inclusive": ("lzw_parse", _mut_parse("cap_inclusive")),
    "budget_off_by_one": ("lzw_parse", _mut_parse("budget_off_by_one")),
    "no_lookup": ("lzw_parse", _mut_parse("no_lookup")),
    "lz78_restart": ("lzw_parse", _mut_parse("lz78_restart")),
    "uniform_remainder_high": ("uniform", _mut_uniform_high),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_allocation_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    if attr == "lzw_parse":
        monkeypatch.setattr(A, "lzw", lambda *a: fn(*a)[0])
    failures = []
    for pin in ALL_PINS:
        try:
            pin(A)
        except Exception as e:  # noqa: BLE001 - any failure counts
            failures.append(f"{pin.__name__}: {type(e).__name__}")
    assert failures, f"mutant {name} passed every pin"


# ---------------------------------------------------- library vs oracle ---
@pytest.fixture(scope="module")
def L():
    from static_token_routed_id_amd import _lib
    return _lib


CASES = [
    # vocab, corpus tokens, budget, k_max, corpus seed
    (256, 20000, 2048, 32, 1),        # the tiny workload's shape
    (1024, 200000, 16384, 64, 2),     # budget reached before the end
    (1024, 50000, 1024 * 512, 512, 3),  # corpus ends first
    (64, 100000, 64 * 8, 8, 4),       # caps reached
    (4096, 300000, 4096 * 4, 512, 5),
    (3, 1000, 3, 1, 6),               # budget = vocab: nothing added
]


@pytest.mark.parametrize("vocab,n,budget,cap,seed", CASES)
def test_lzw_matches_oracle(L, vocab, n, budget, cap, seed):
    corpus = wl.synthetic_corpus(vocab, n, seed=seed)
    counts, offsets = L.l3_allocate(L.L3_ALLOC_LZW, corpus, vocab, budget, cap)
    want = A.lzw(corpus, vocab, budget, cap)
    assert np.array_equal(counts, want)
    assert np.array_equal(offsets, A.offsets(want))
    assert counts.min() >= 1 and counts.max() <= cap


def test_lzw_textbook(L):
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "lzw_textbook.json")))
    sym = g["symbols"]
    corpus = np.asarray([sym.index(ch) for ch in g["text"]], np.int32)
    for case in g["cases"]:
        counts, _ = L.l3_allocate(L.L3_ALLOC_LZW, corpus, len(sym),
                                  case["budget"], case["k_max"])
        assert list(counts) == [case["counts"][ch] for ch in sym], case["name"]


def test_lzw_empty_and_single(L):
    for corpus in (np.zeros(0, np.int32), np.array([3], np.int32)):
        counts, offsets = L.l3_allocate(L.L3_ALLOC_LZW, corpus, 8, 40, 8)
        assert np.array_equal(counts, A.lzw(corpus, 8, 40, 8))
        assert list(counts) == [1] * 8 and offsets[-1] == 8


@pytest.mark.parametrize("vocab,budget,cap", [(7, 7, 3), (7, 20, 3),
                                              (131072, 1 << 22, 512),
                                              (1000, 5555, 8)])
def test_uniform_matches_oracle(L, vocab, budget, cap):
    counts, offsets = L.l3_allocate(L.L3_ALLOC_UNIFORM, None, vocab, budget,
                                    cap)
    want = A.uniform(vocab, budget, cap)
    assert np.array_equal(counts, want)
    assert np.array_equal(offsets, A.offsets(want))


def test_allocate_errors(L):
    c = np.array([0, 1, 2], np.int32)
    bad = [(L.L3_ALLOC_LZW, np.array([0, 9], np.int32), 5, 10, 4,
            L.L3_ERR_TOKEN_RANGE),
           (L.L3_ALLOC_LZW, np.array([-1], np.int32), 5, 10, 4,
            L.L3_ERR_TOKEN_RANGE),
           (L.L3_ALLOC_LZW, c, 5, 4, 4, L.L3_ERR_SHAPE),      # budget < V
           (L.L3_ALLOC_LZW, c, 5, 21, 4, L.L3_ERR_SHAPE),     # budget > V k
           (L.L3_ALLOC_LZW, c, 5, 10, 0, L.L3_ERR_SHAPE),     # k < 1
           (L.L3_ALLOC_LZW, c, 5, 10, 513, L.L3_ERR_SHAPE),   # k > 512
           (L.L3_ALLOC_UNIFORM, c, 0, 10, 4, L.L3_ERR_SHAPE),  # V < 1
           (7, c, 5, 10, 4, L.L3_ERR_DTYPE)]                  # method
    for method, corpus, vocab, budget, cap, code in bad:
        with pytest.raises(L.L3Error) as e:
            L.l3_allocate(method, corpus, vocab, budget, cap)
        assert e.value.status == code, (method, vocab, budget, cap)
    lib = L.lib()
    assert lib.l3_allocate(L.L3_ALLOC_LZW, None, 0, 5, 10, 4, None,
                           None) == L.L3_ERR_NULL
