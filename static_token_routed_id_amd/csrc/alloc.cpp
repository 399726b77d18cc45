// Embedding allocation: how many rows of K and V each token id owns
// (gist.science explainer of "L^3: Large Lookup Layers", Technical Summary,
// Information-Theoretic Embedding Allocation: a budget of embeddings spread
// over the vocabulary by an LZW-variant scan of a corpus, frequent context
// suffixes getting more embeddings, every token between 1 and k; Key
// Contributions: compared with a uniform allocation).
//
// Host code. The scan is LZW's parse, a chain in which every step depends
// on the dictionary the previous steps built, so it runs once per model on
// one CPU core, before any batch is planned; its output is the offsets
// array l3_plan takes. The dictionary is a trie held in an open-addressing
// hash table keyed by (node, next token).
//
// The pages give no steps; the reading implemented (each point a choice):
//   the dictionary starts with every single token (each token owns one
//   embedding); the corpus is parsed as LZW parses it (the phrase grows while
//   phrase + next token is in the dictionary, else phrase + next token c is
//   added and the next phrase starts at c); an added entry is one more
//   embedding of its last token c (context suffix, then c); a token that
//   owns k_max embeddings takes no new entry; the scan stops when the
//   entries reach the budget, or at the end of the corpus.
// Uniform: budget // vocab each, the remainder one each to the lowest ids.

#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "l3.h"

namespace {

// Open-addressing map from a 64-bit key to a node id (linear probing; the
// key ~0 marks an empty slot, which no (node, token) key can equal).
class NodeMap {
 public:
  explicit NodeMap(int64_t max_entries) {
    size_t cap = 1024;
    while (cap < static_cast<size_t>(2 * max_entries + 16)) cap <<= 1;
    keys_.assign(cap, ~uint64_t(0));
    vals_.assign(cap, 0);
    mask_ = cap - 1;
  }
  // node id, or -1
  int64_t find(uint64_t key) const {
    for (size_t i = hash(key) & mask_;; i = (i + 1) & mask_) {
      if (keys_[i] == key) return vals_[i];
      if (keys_[i] == ~uint64_t(0)) return -1;
    }
  }
  void insert(uint64_t key, int64_t node) {
    size_t i = hash(key) & mask_;
    while (keys_[i] != ~uint64_t(0)) i = (i + 1) & mask_;
    keys_[i] = key;
    vals_[i] = node;
  }

 private:
  static size_t hash(uint64_t k) {
    k ^= k >> 33;
    k *= 0xff51afd7ed558ccdULL;
    k ^= k >> 33;
    k *= 0xc4ceb9fe1a85ec53ULL;
    k ^= k >> 33;
    return static_cast<size_t>(k);
  }
  std::vector<uint64_t> keys_;
  std::vector<int64_t> vals_;
  size_t mask_ = 0;
};

void uniform_counts(int64_t vocab, int64_t budget, int k_max,
                    int64_t* counts) {
  const int64_t q = budget / vocab, r = budget % vocab;
  for (int64_t t = 0; t < vocab; ++t) {
    int64_t v = q + (t < r ? 1 : 0);
    counts[t] = v < 1 ? 1 : (v > k_max ? k_max : v);
  }
}

void lzw_counts(const int32_t* corpus, int64_t n, int64_t vocab,
                int64_t budget, int k_max, int64_t* counts) {
  for (int64_t t = 0; t < vocab; ++t) counts[t] = 1;
  if (n == 0) return;
  int64_t total = vocab;
  const int64_t max_entries = budget - vocab;
  NodeMap map(max_entries);
  int64_t next = vocab;  // node ids 0 .. vocab - 1 are the single tokens
  int64_t w = corpus[0];
  const uint64_t V = static_cast<uint64_t>(vocab);
  for (int64_t i = 1; i < n; ++i) {
    if (total >= budget) break;
    const int64_t c = corpus[i];
    const uint64_t key = static_cast<uint64_t>(w) * V + static_cast<uint64_t>(c);
    const int64_t hit = map.find(key);
    if (hit >= 0) {
      w = hit;
      continue;
    }
    if (counts[c] < k_max) {
      map.insert(key, next++);
      ++counts[c];
      ++total;
    }
    w = c;
  }
}

}  // namespace

extern "C" {

l3_status l3_allocate(int method, const int32_t* corpus, int64_t n_tokens,
                      int64_t vocab, int64_t budget, int32_t k_max,
                      int64_t* counts, int64_t* offsets) {
  try {
    if (method != L3_ALLOC_UNIFORM && method != L3_ALLOC_LZW)
      return L3_ERR_DTYPE;
    if (!counts) return L3_ERR_NULL;
    if (vocab < 1 || vocab > (int64_t(1) << 31) - 2 || k_max < 1 ||
        k_max > L3_MAX_ROWS_PER_ID || n_tokens < 0 || budget < vocab ||
        budget > vocab * k_max)
      return L3_ERR_SHAPE;
    if (method == L3_ALLOC_LZW) {
      if (n_tokens > 0 && !corpus) return L3_ERR_NULL;
      for (int64_t i = 0; i < n_tokens; ++i)
        if (corpus[i] < 0 || corpus[i] >= vocab) return L3_ERR_TOKEN_RANGE;
      lzw_counts(corpus, n_tokens, vocab, budget, k_max, counts);
    } else {
      uniform_counts(vocab, budget, k_max, counts);
    }
    if (offsets) {
      offsets[0] = 0;
      for (int64_t t = 0; t < vocab; ++t) offsets[t + 1] = offsets[t] + counts[t];
    }
    return L3_OK;
  } catch (const std::bad_alloc&) {
    return L3_ERR_WORKSPACE;
  } catch (...) {
    return L3_ERR_HIP;
  }
}

}  // extern "C"
