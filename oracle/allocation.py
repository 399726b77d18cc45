"""CPU oracle of the embedding allocation of the L3 layer.

TEST INFRASTRUCTURE ONLY. This module is the slow, obviously-correct
statement of how a budget of embedding rows is spread over the vocabulary;
the C++ allocator in libl3 (l3_allocate) is checked against it bit for bit.
Only the tests and the benchmark's CPU-baseline leg may import it. It shares
no code with the library and imports nothing from it.

Source (gist.science explainer of "L^3: Large Lookup Layers", Technical
Summary, Information-Theoretic Embedding Allocation; Key Contributions):
  * a fixed budget v of embeddings is spread over the vocabulary by a
    variant of the LZW compression algorithm that scans a corpus for
    frequent suffixes of contexts; frequent context suffixes get more
    embeddings (allocation as the dual of lossless compression);
  * every token gets at least one and at most k embeddings (k = 512 in the
    pages' example);
  * the result is heavy-tailed; the pages compare it with a uniform
    allocation.

The pages give no steps of the algorithm, so what follows is a reading,
the plainest LZW the description supports (each point is a choice):
  A1 the dictionary starts with every single token, so every token owns
     one embedding before the scan (the lower bound 1);
  A2 the corpus is parsed as LZW parses it: the current phrase w grows while
     w + c is in the dictionary; otherwise w + c is a new entry and the next
     phrase starts at c;
  A3 a new entry w + c is the context suffix w followed by token c, so it is
     one more embedding of token c (the token whose rows the layer reads
     when c is the current token);
  A4 a token that already owns k embeddings takes no new entry (w + c is not
     added; the parse still restarts at c) -- the upper bound k;
  A5 the scan stops when the entries reach the budget v (or at the end of
     the corpus, one pass); budget left over stays unassigned, so
     sum(n_t) = min(v, V + entries added);
  A6 uniform baseline: q = v // V, r = v % V; token t gets q + (t < r),
     clamped to [1, k].
Parity of A1-A6 against the pages is unpinned: the pages print neither the
steps nor any allocation to compare with. The tests pin this oracle to the
LZW definition itself (a hand-worked parse of a textbook string, the parse
reproducing the corpus, each entry extending a parsed phrase by the next
phrase's first token) and to the bounds above.
"""
from __future__ import annotations

from typing import Dict, List, Tuple

import numpy as np


class AllocationInputError(ValueError):
    """Raised for inputs the allocation does not define."""


def _check(vocab: int, budget: int, k_max: int) -> None:
    if vocab < 1:
        raise AllocationInputError("vocab must be >= 1")
    if k_max < 1:
        raise AllocationInputError("k_max must be >= 1")
    if budget < vocab:
        raise AllocationInputError("budget below one embedding per token")
    if budget > vocab * k_max:
        raise AllocationInputError("budget above k_max embeddings per token")


def uniform(vocab: int, budget: int, k_max: int) -> np.ndarray:
    """Reading A6: the budget split evenly, the remainder to the lowest ids."""
    _check(vocab, budget, k_max)
    q, r = divmod(int(budget), int(vocab))
    n = [q + (1 if t < r else 0) for t in range(vocab)]
    return np.asarray([min(max(v, 1), k_max) for v in n], dtype=np.int64)


def lzw_parse(corpus, vocab: int, budget: int,
              k_max: int) -> Tuple[np.ndarray, List[Tuple[int, ...]],
                                   List[Tuple[int, ...]]]:
    """Readings A1-A5. Returns (counts [vocab] int64, entries added in
    order (each a tuple of tokens), the parse (the phrases the corpus was
    cut into, in order; the last one may be the unfinished phrase at the
    end of the scan))."""
    _check(vocab, budget, k_max)
    toks = [int(t) for t in np.asarray(corpus).reshape(-1)]
    for t in toks:
        if t < 0 or t >= vocab:
            raise AllocationInputError(f"token {t} outside [0, {vocab})")
    counts = [1] * vocab                       # A1
    dictionary: Dict[Tuple[int, ...], bool] = {(t,): True
                                               for t in range(vocab)}
    entries: List[Tuple[int, ...]] = []
    parse: List[Tuple[int, ...]] = []
    total = vocab
    if not toks:
        return np.asarray(counts, np.int64), entries, parse
    w: Tuple[int, ...] = (toks[0],)
    for c in toks[1:]:
        if total >= budget:                    # A5: budget reached
            break
        wc = w + (c,)
        if wc in dictionary:                   # A2: the phrase grows
            w = wc
            continue
        parse.append(w)
        if counts[c] < k_max:                  # A4: cap
            dictionary[wc] = True              # A3: one more row of c
            entries.append(wc)
            counts[c] += 1
            total += 1
        w = (c,)                               # A2: next phrase starts at c
    parse.append(w)
    return np.asarray(counts, np.int64), entries, parse


def lzw(corpus, vocab: int, budget: int, k_max: int) -> np.ndarray:
    """Rows per token id from the LZW-variant scan (readings A1-A5)."""
    return lzw_parse(corpus, vocab, budget, k_max)[0]


def offsets(counts) -> np.ndarray:
    """CSR offsets: the exclusive prefix sum of the counts (length V + 1)."""
    c = [int(v) for v in np.asarray(counts).reshape(-1)]
    out = [0]
    for v in c:
        out.append(out[-1] + v)
    return np.asarray(out, dtype=np.int64)
