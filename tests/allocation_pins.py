"""Pins of the allocation oracle (oracle/allocation.py): checks against facts
that do not come from it. Each takes the module ``A`` and raises
AssertionError on a disagreement; tests/test_allocation.py runs them on the
oracle and on planted mistakes.

Facts used:
  * LZW as Welch defined it (IEEE Computer, 1984), worked by hand on a
    textbook string (tests/golden/lzw_textbook.json), with and without a cap
    and a budget;
  * properties every LZW parse has: the phrases concatenate to the scanned
    corpus; every phrase was in the dictionary when it ended; the phrase
    extended by the next phrase's first token was not (greedy longest
    match); each added entry is exactly that extension;
  * the bounds the pages state (Information-Theoretic Embedding Allocation,
    Constraints): every token between 1 and k embeddings, the total within
    the budget; a heavy tail on a Zipf corpus (Result);
  * the uniform split in closed form.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _corpus(seed, vocab, n, zipf_s=1.0, max_len=4):
    """A small seeded corpus with repeated phrases (numpy only)."""
    g = np.random.default_rng(seed)
    f = 1.0 / np.arange(1, vocab + 1) ** zipf_s
    f /= f.sum()
    book = [g.choice(vocab, size=int(g.integers(1, max_len + 1)), p=f)
            for _ in range(4 * vocab)]
    pf = 1.0 / np.arange(1, len(book) + 1) ** zipf_s
    pf /= pf.sum()
    out = []
    while len(out) < n:
        out.extend(int(t) for t in book[int(g.choice(len(book), p=pf))])
    return np.asarray(out[:n], np.int32)


def pin_textbook(A):
    g = json.load(open(os.path.join(GOLDEN, "lzw_textbook.json")))
    sym = g["symbols"]
    enc = lambda s: tuple(sym.index(ch) for ch in s)
    corpus = np.asarray(enc(g["text"]), np.int32)
    for case in g["cases"]:
        counts, entries, parse = A.lzw_parse(corpus, len(sym), case["budget"],
                                             case["k_max"])
        assert [tuple(e) for e in entries] == [enc(e) for e in case["entries"]], \
            f"{case['name']}: entries"
        assert [tuple(p) for p in parse] == [enc(p) for p in case["parse"]], \
            f"{case['name']}: parse"
        want = [case["counts"][ch] for ch in sym]
        assert list(counts) == want, f"{case['name']}: counts"


def _cases():
    out = []
    for seed, (vocab, n, cap) in enumerate([(5, 300, 512), (12, 2000, 6),
                                            (40, 5000, 3), (8, 1500, 512)]):
        out.append((seed, vocab, n, cap))
    return out


def pin_parse_properties(A):
    for seed, vocab, n, cap in _cases():
        corpus = _corpus(100 + seed, vocab, n)
        for budget in (vocab, vocab + 7, vocab * cap // 2 + 1, vocab * cap):
            budget = max(vocab, min(budget, vocab * cap))
            counts, entries, parse = A.lzw_parse(corpus, vocab, budget, cap)
            flat = [t for p in parse for t in p]
            assert flat == [int(t) for t in corpus[:len(flat)]], \
                "phrases concatenate to the scanned corpus"
            if sum(counts) < budget:
                assert len(flat) == n, "the whole corpus is scanned"
            dictionary = {(t,) for t in range(vocab)}
            per_token = [1] * vocab
            added = []
            for j, ph in enumerate(parse):
                assert tuple(ph) in dictionary, "a phrase not in the dictionary"
                if j + 1 == len(parse):
                    break
                cand = tuple(ph) + (parse[j + 1][0],)
                assert cand not in dictionary, "the match was not the longest"
                c = cand[-1]
                if per_token[c] < cap and len(added) + vocab < budget:
                    dictionary.add(cand)
                    added.append(cand)
                    per_token[c] += 1
            assert [tuple(e) for e in entries] == added, \
                "entries are the parse's extensions, in order"
            assert list(counts) == per_token, "one embedding per entry's last token"


def pin_bounds(A):
    for seed, vocab, n, cap in _cases():
        corpus = _corpus(200 + seed, vocab, n)
        for budget in (vocab + 3, vocab * cap):
            c = A.lzw(corpus, vocab, budget, cap)
            assert c.min() >= 1 and c.max() <= cap, "1 <= n_t <= k"
            assert c.sum() <= budget, "within the budget"
            off = A.offsets(c)
            assert off[0] == 0 and np.array_equal(np.diff(off), c)
    # a long corpus reaches a small budget exactly
    corpus = _corpus(7, 20, 20000)
    assert A.lzw(corpus, 20, 20 * 10 // 2, 10).sum() == 100


def pin_heavy_tail(A):
    """Zipf corpus (frequency rank = id): the most frequent ids get many
    embeddings, the rare ones few (the pages' Result)."""
    corpus = _corpus(3, 200, 60000, zipf_s=1.1)
    c = A.lzw(corpus, 200, 200 * 64 // 4, 64)
    assert c[:5].mean() >= 8 * np.median(c), "not heavy-tailed"
    assert c[0] > c[-50:].mean()


def pin_uniform(A):
    for vocab, budget, cap in ((7, 7, 3), (7, 20, 3), (7, 21, 3), (10, 99, 512),
                               (1, 1, 1), (1000, 5555, 8)):
        c = A.uniform(vocab, budget, cap)
        q, r = divmod(budget, vocab)
        assert c.sum() == budget
        assert list(c[:r]) == [q + 1] * r and list(c[r:]) == [q] * (vocab - r)


def pin_errors(A):
    bad = [(np.array([0, 5], np.int32), 5, 10, 4),   # token outside [0, V)
           (np.array([0], np.int32), 5, 4, 4),        # budget < V
           (np.array([0], np.int32), 5, 21, 4),       # budget > V k
           (np.array([0], np.int32), 5, 5, 0),        # k < 1
           (np.array([0], np.int32), 0, 5, 4)]        # V < 1
    for corpus, vocab, budget, cap in bad:
        try:
            A.lzw(corpus, vocab, budget, cap)
        except A.AllocationInputError:
            continue
        raise AssertionError(f"accepted V={vocab} budget={budget} k={cap}")


ALL_PINS = [pin_textbook, pin_parse_properties, pin_bounds, pin_heavy_tail,
            pin_uniform, pin_errors]
