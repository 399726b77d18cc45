// Plan: sort the batch by token id and cut it into one segment per id.
//
// gist.science explainer of "L^3: Large Lookup Layers", Technical Summary,
// Systems-Friendly Design, Batch Sorting: sorting the tokens of a batch by id
// makes the layer's attention mask block-diagonal, i.e. every token of one id
// attends over the same rows K_t, V_t. Core Architecture, Static Routing: the
// rows of id t are known from t alone (here: offsets[t] .. offsets[t+1]-1),
// and Information-Theoretic Embedding Allocation, Constraints: each id owns
// between 1 and k rows, which the plan checks for every id that occurs.
//
// The sort key is (id, position), unique, so every correct sort gives the
// same permutation. Three implementations:
//   * batches up to 64 tokens (decode): one wavefront, the sort, the
//     segments and the item map by cross-lane operations (no barrier);
//   * batches up to 4096 tokens: one 1024-thread workgroup, bitonic sort of
//     64-bit keys (up to 1024 tokens one key a thread in registers, the
//     partners in a wavefront by shuffles; above, in LDS), then segment
//     cut, work-item count and (without group items) the wave items' map
//     in the same launch (one launch: such batches are latency bound);
//   * larger batches: LSD radix sort of the 32-bit ids with the position as
//     payload (stable, 8- or 9-bit digits; per digit a histogram of each
//     1024-key tile, then a ranked scatter whose workgroups take their
//     offsets from all the tiles' counts), then segment cut kernels.
// After the segments, the plan counts the forward pass's work items: a
// segment with n_g >= group_min_rows (large batches only) yields one group
// item if m_g <= 64, else ceil(m_g / 128) (seg_gitem_start), any other
// segment ceil(m_g / 16) * ceil(n_g / chunk) wave items (seg_item_start);
// both are exclusive prefix sums.

#include "l3_device.h"
#include "l3_internal.h"

namespace l3 {

// Record a bad id / bad row count, read one id's rows. Returns false if the
// id is unusable.
__device__ __forceinline__ bool id_rows(const PlanParams& p, int t,
                                        int64_t* r0, int* n,
                                        int32_t* header) {
  if (t < 0 || t >= p.vocab) {
    atomicOr(&header[0], kBadId);
    *r0 = 0;
    *n = 1;
    return false;
  }
  int64_t a = p.offsets[t], b = p.offsets[t + 1];
  int64_t cnt = b - a;
  if (cnt < 1 || cnt > p.k_max || a < 0 || b > p.rows) {
    atomicOr(&header[0], kBadCount);
    *r0 = 0;
    *n = 1;
    return false;
  }
  *r0 = a;
  *n = static_cast<int>(cnt);
  return true;
}

// Segments with at least group_min_rows rows (when enabled) go to the
// workgroup-per-item group kernel: one item if they have at most kGroupTok
// tokens, else items of kHotTok tokens; the others go to the wave kernel in
// tiles of kTokTile tokens times row chunks.
__device__ __forceinline__ bool is_group(int n, const PlanParams& p) {
  return p.group_min_rows > 0 && n >= p.group_min_rows;
}
__device__ __forceinline__ int items_of(int m, int n, const PlanParams& p) {
  return is_group(n, p) ? 0 : ceil_div(m, kTokTile) * ceil_div(n, p.chunk_rows);
}
// wave items of a segment when every id goes to the wave kernel
__device__ __forceinline__ int aitems_of(int m, int n, const PlanParams& p) {
  return ceil_div(m, kTokTile) * ceil_div(n, p.chunk_rows);
}
__device__ __forceinline__ int gitems_of(int m, int n, const PlanParams& p) {
  if (!is_group(n, p)) return 0;
  return m > kGroupTok ? ceil_div(m, kHotTok) : 1;
}

// ----------------------------------------------------------------- tiny ---
// Batches of at most 64 tokens without group items (decode): the whole plan
// on one wavefront, token i on lane i, with no workgroup barrier: bitonic
// sort of the (id, position) keys across the lanes by shuffles, segment
// starts from a ballot of id changes, the wave items' exclusive scan by
// shuffles, and each segment's lane writes its segment and its items' map.
// The id and row-count checks are ballots, so the status is known in
// registers: the header is written once at the end, and the kernel waits
// on global memory only for the ids and for the row ranges.
constexpr int kTinyPlanMax = 64;
static_assert(kHeaderInts <= 64, "one lane a header word");
__global__ __launch_bounds__(64) void plan_tiny_kernel(PlanDev pd,
                                                       PlanParams p) {
  const int lane = threadIdx.x;
  const int B = p.B;
  unsigned long long key = ~0ull;
  bool bad_id = false;
  if (lane < B) {
    const int t = p.ids[lane];
    bad_id = t < 0 || t >= p.vocab;
    key = (static_cast<unsigned long long>(static_cast<uint32_t>(t)) << 32) |
          static_cast<uint32_t>(lane);
  }
  // bitonic sort, ascending (padding keys ~0 sort last)
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const unsigned long long other = __shfl_xor(key, stride);
      const bool up = (lane & size) == 0;
      const bool low = (lane & stride) == 0;
      const unsigned long long mn = key < other ? key : other;
      const unsigned long long mx = key < other ? other : key;
      key = (low == up) ? mn : mx;
    }
  }
  const int t = static_cast<int>(key >> 32);
  const int tprev = __shfl_up(t, 1);
  const bool start = lane < B && (lane == 0 || t != tprev);
  if (lane < B) {
    pd.perm[lane] = static_cast<int>(key & 0xffffffffu);
    pd.sorted_ids[lane] = t;
  }
  const unsigned long long starts = __ballot(start);
  const int S = __popcll(starts);
  const unsigned long long below = (1ull << lane) - 1;
  const int sidx = __popcll(starts & below);  // segment of a start lane
  // tokens of the segment starting here: up to the next start, or B
  const unsigned long long after = lane < 63 ? starts >> (lane + 1) : 0ull;
  const int next = after ? lane + 1 + __ffsll(after) - 1 : B;
  int n = 1, items = 0;
  bool bad_count = false;
  if (start) {
    // the id's rows (a bad id keeps row 0 and one row, as the other plans)
    int64_t r0 = 0;
    if (t >= 0 && t < p.vocab) {
      const int64_t a = p.offsets[t], b = p.offsets[t + 1];
      const int64_t c = b - a;
      if (c < 1 || c > p.k_max || a < 0 || b > p.rows) {
        bad_count = true;
      } else {
        r0 = a;
        n = static_cast<int>(c);
      }
    }
    pd.seg_id[sidx] = t;
    pd.seg_tok_start[sidx] = lane;
    pd.seg_row_off[sidx] = r0;
    pd.seg_n[sidx] = n;
    items = aitems_of(next - lane, n, p);
  }
  const int status = (__ballot(bad_id) ? kBadId : 0) |
                     (__ballot(bad_count) ? kBadCount : 0);
  const int incl = wave_incl_scan(items, lane);
  const int total = __shfl(incl, 63);
  const int w0 = incl - items;
  if (start) {
    pd.seg_item_start[sidx] = w0;
    pd.seg_gitem_start[sidx] = 0;
  }
  if (lane == 0) {
    pd.seg_tok_start[S] = B;
    pd.seg_item_start[S] = total;
    pd.seg_gitem_start[S] = 0;
  }
  // status, segment and item counts; every queue and other count zero
  if (lane < kHeaderInts)
    pd.header[lane] = lane == 0                 ? status
                      : lane == 1               ? S
                      : lane == 2 || lane == 8  ? total
                                                : 0;
  // the items' map, unless an id or a row count was bad (as item_map_kernel)
  if (status == 0 && start)
    for (int i = 0; i < items; ++i)
      pd.item_map[w0 + i] = make_int2(sidx, i);
}

// ---------------------------------------------------------------- small ---
__global__ __launch_bounds__(1024) void plan_small_kernel(PlanDev pd,
                                                          PlanParams p) {
  __shared__ unsigned long long keys[kSmallPlanMax];
  __shared__ int tmp[1024 / 64 + 1];
  // the checks' verdict (kBadId | kBadCount), gathered in LDS; the header
  // is written once, after the scans
  __shared__ int s_status;
  const int tid = threadIdx.x;
  const int B = p.B;
  int B2 = 1;
  while (B2 < B) B2 <<= 1;
  if (tid == 0) s_status = 0;
  __syncthreads();

  if (B2 <= 1024) {
    // one key a thread: bitonic sort, ascending, in registers; partners
    // within the wavefront (stride < 64) by shuffles, the others through
    // LDS (padding keys ~0 sort last)
    unsigned long long key = ~0ull;
    if (tid < B) {
      const int t = p.ids[tid];
      if (t < 0 || t >= p.vocab) atomicOr(&s_status, kBadId);
      key = (static_cast<unsigned long long>(static_cast<uint32_t>(t))
             << 32) |
            static_cast<uint32_t>(tid);
    }
    for (int size = 2; size <= B2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        unsigned long long other;
        if (stride >= 64) {
          if (tid < B2) keys[tid] = key;
          __syncthreads();
          other = tid < B2 ? keys[tid ^ stride] : key;
          __syncthreads();
        } else {
          other = __shfl_xor(key, stride);
        }
        const bool up = (tid & size) == 0;
        const bool low = (tid & stride) == 0;
        const unsigned long long mn = key < other ? key : other;
        const unsigned long long mx = key < other ? other : key;
        key = (low == up) ? mn : mx;
      }
    }
    if (tid < B2) keys[tid] = key;
    __syncthreads();
  } else {
    for (int i = tid; i < B2; i += 1024) {
      unsigned long long k = ~0ull;
      if (i < B) {
        int t = p.ids[i];
        if (t < 0 || t >= p.vocab) atomicOr(&s_status, kBadId);
        k = (static_cast<unsigned long long>(static_cast<uint32_t>(t))
             << 32) |
            static_cast<uint32_t>(i);
      }
      keys[i] = k;
    }
    __syncthreads();
    // bitonic sort, ascending, in LDS
    for (int size = 2; size <= B2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < (B2 >> 1); i += 1024) {
          int lo = 2 * i - (i & (stride - 1));
          int hi = lo + stride;
          bool up = (lo & size) == 0;
          unsigned long long a = keys[lo], b = keys[hi];
          if ((a > b) == up) {
            keys[lo] = b;
            keys[hi] = a;
          }
        }
        __syncthreads();
      }
    }
  }
  // perm, sorted ids; segment flags scanned in contiguous chunks per thread
  const int per = ceil_div(B, 1024);
  const int j0 = min(B, tid * per), j1 = min(B, j0 + per);
  int cnt = 0;
  for (int j = j0; j < j1; ++j) {
    unsigned long long k = keys[j];
    int t = static_cast<int>(k >> 32);
    pd.perm[j] = static_cast<int>(k & 0xffffffffu);
    pd.sorted_ids[j] = t;
    cnt += (j == 0 || t != static_cast<int>(keys[j - 1] >> 32)) ? 1 : 0;
  }
  int total;
  int s = block_excl_scan<1024>(cnt, tmp, &total);
  const int S = total;
  for (int j = j0; j < j1; ++j) {
    int t = static_cast<int>(keys[j] >> 32);
    if (j == 0 || t != static_cast<int>(keys[j - 1] >> 32)) {
      int64_t r0;
      int n;
      id_rows(p, t, &r0, &n, &s_status);
      pd.seg_id[s] = t;
      pd.seg_tok_start[s] = j;
      pd.seg_row_off[s] = r0;
      pd.seg_n[s] = n;
      ++s;
    }
  }
  if (tid == 0) pd.seg_tok_start[S] = B;
  __syncthreads();
  // work items per segment (wave items and group items), exclusive scans
  const int sper = ceil_div(S, 1024);
  const int s0 = min(S, tid * sper), s1 = min(S, s0 + sper);
  int icnt = 0, gcnt = 0, acnt = 0;
  for (int g = s0; g < s1; ++g) {
    const int m = pd.seg_tok_start[g + 1] - pd.seg_tok_start[g];
    icnt += items_of(m, pd.seg_n[g], p);
    gcnt += gitems_of(m, pd.seg_n[g], p);
    acnt += aitems_of(m, pd.seg_n[g], p);
  }
  int ibase = block_excl_scan<1024>(icnt, tmp, &total);
  int gtotal, atotal;
  int gbase = block_excl_scan<1024>(gcnt, tmp, &gtotal);
  int abase = block_excl_scan<1024>(acnt, tmp, &atotal);
  for (int g = s0; g < s1; ++g) {
    const int m = pd.seg_tok_start[g + 1] - pd.seg_tok_start[g];
    pd.seg_item_start[g] = ibase;
    pd.seg_gitem_start[g] = gbase;
    if (p.group_min_rows > 0) pd.seg_aitem_start[g] = abase;
    ibase += items_of(m, pd.seg_n[g], p);
    gbase += gitems_of(m, pd.seg_n[g], p);
    abase += aitems_of(m, pd.seg_n[g], p);
  }
  if (tid == 0) {
    pd.seg_item_start[S] = total;
    pd.seg_gitem_start[S] = gtotal;
    if (p.group_min_rows > 0) pd.seg_aitem_start[S] = atotal;
  }
  // status (every check precedes the scans' barriers), segment and item
  // counts; every queue and other count zero
  const int status = s_status;
  if (tid < kHeaderInts)
    pd.header[tid] = tid == 0                ? status
                     : tid == 1              ? S
                     : tid == 2              ? total
                     : tid == 3              ? gtotal
                     : tid == 8              ? atotal
                                             : 0;
  // Without group items (the group kernel is off at these sizes) the wave
  // items' map is the only one, and it is written here, one wave per
  // segment as item_map_kernel does, which saves that launch; nothing is
  // written for a plan with a bad id or row count (as there).
  if (p.group_min_rows == 0) {
    __syncthreads();  // every segment's item start is written
    if (status == 0) {
      const int lane = tid & 63;
      for (int g = tid >> 6; g < S; g += 1024 / 64) {
        const int w0 = pd.seg_item_start[g], w1 = pd.seg_item_start[g + 1];
        for (int i = w0 + lane; i < w1; i += 64)
          pd.item_map[i] = make_int2(g, i - w0);
      }
    }
  }
}

// ---------------------------------------------------------------- large ---
// Digit histogram of one 1024-key tile (DB-bit digits, 2^DB buckets);
// pass 0 also checks the id range and records the tile's verdict in
// bad[tile] (kBadId or 0), which the first scatter folds into the header.
template <int DB>
__global__ __launch_bounds__(256) void radix_hist_kernel(
    const int32_t* kin, int B, int shift, int32_t* hist, int nblk,
    int64_t vocab, int32_t* bad) {
  constexpr int NB = 1 << DB;
  __shared__ int h[NB];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  for (int q = tid; q < NB; q += 256) h[q] = 0;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  for (int r = 0; r < kSortTile / 256; ++r) {
    int i = blockIdx.x * kSortTile + r * 256 + tid;
    if (i < B) {
      int k = kin[i];
      if (bad && (k < 0 || k >= vocab)) s_bad = kBadId;
      atomicAdd(&h[(static_cast<uint32_t>(k) >> shift) & (NB - 1u)], 1);
    }
  }
  __syncthreads();
  for (int q = tid; q < NB; q += 256) hist[q * nblk + blockIdx.x] = h[q];
  if (bad && tid == 0) bad[blockIdx.x] = s_bad;
}

// In-place exclusive scan of a[0..n) by one 1024-thread workgroup: rounds
// of 16384 values, each thread taking 16 consecutive ones (all loads of a
// round in flight together), one workgroup scan per round. Returns the total.
__device__ int scan_excl_1024(int32_t* a, int n, int* tmp) {
  const int tid = threadIdx.x;
  int carry = 0;
  for (int base = 0; base < n; base += 16 * 1024) {
    const int i0 = base + tid * 16;
    int v[16];
    if (i0 + 16 <= n) {
      // whole run of 16: four 16-byte loads (a is 256-byte aligned)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int4 q = *reinterpret_cast<const int4*>(a + i0 + 4 * j);
        v[4 * j] = q.x;
        v[4 * j + 1] = q.y;
        v[4 * j + 2] = q.z;
        v[4 * j + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = i0 + j < n ? a[i0 + j] : 0;
    }
    int sum = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int t = v[j];
      v[j] = sum;
      sum += t;
    }
    int total;
    const int off = block_excl_scan<1024>(sum, tmp, &total) + carry;
    if (i0 + 16 <= n) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<int4*>(a + i0 + 4 * j) =
            make_int4(v[4 * j] + off, v[4 * j + 1] + off, v[4 * j + 2] + off,
                      v[4 * j + 3] + off);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (i0 + j < n) a[i0 + j] = v[j] + off;
    }
    carry += total;
  }
  return carry;
}

// Stable scatter of one 1024-key tile by one DB-bit digit. The tile's first
// output position for each digit (every key of a smaller digit, and this
// digit's keys in earlier tiles) comes from the raw per-tile counts
// hist[digit * nblk + tile]: each workgroup reads them all (L2-resident)
// instead of waiting for a separate scan. Keys of a tile are taken in
// order, 256 at a time; within a wave the rank among equal digits comes
// from a ballot match on the digit bits, across waves from LDS counts.
template <int DB>
__global__ __launch_bounds__(256) void radix_scatter_kernel(
    const int32_t* kin, const int32_t* vin, int32_t* kout, int32_t* vout,
    int B, int shift, const int32_t* hist, int nblk, int32_t* header,
    const int32_t* bad) {
  constexpr int NB = 1 << DB;
  constexpr int DPT = NB / 256;  // digits a thread, consecutive
  __shared__ int base[NB];
  __shared__ int wcnt[4][NB];
  __shared__ int tmp[256 / 64 + 1];
  __shared__ int s_bad;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int me = blockIdx.x;
  if (header && me == 0) {
    // first pass: the plan's header starts here (status = the tiles' id
    // checks, every count and queue zero); nothing reads it before the
    // segment kernels
    if (tid == 0) s_bad = 0;
    __syncthreads();
    int f = 0;
    for (int i = tid; i < nblk; i += 256) f |= bad[i];
    if (f) atomicOr(&s_bad, f);
    __syncthreads();
    if (tid < kHeaderInts) header[tid] = tid == 0 ? s_bad : 0;
  }
  // the tile's keys and payloads, loaded first: their latency hides behind
  // the counts' reads
  constexpr int RND = kSortTile / 256;
  int keys[RND], vals[RND];
#pragma unroll
  for (int r = 0; r < RND; ++r) {
    const int i = blockIdx.x * kSortTile + r * 256 + tid;
    keys[r] = i < B ? kin[i] : 0;
    vals[r] = i < B ? (vin ? vin[i] : i) : 0;
  }
  int tot[DPT], pre[DPT], mine = 0;
#pragma unroll
  for (int u = 0; u < DPT; ++u) {
    const int32_t* hq = hist + static_cast<int64_t>(tid * DPT + u) * nblk;
    int t = 0, pr = 0;
    if (nblk % 4 == 0) {
#pragma unroll 16
      for (int b = 0; b < nblk; b += 4) {
        const int4 c = *reinterpret_cast<const int4*>(hq + b);
        const int c4 = c.x + c.y + c.z + c.w;
        t += c4;
        if (b + 4 <= me)
          pr += c4;
        else if (b < me)
          pr += c.x + (b + 1 < me ? c.y : 0) + (b + 2 < me ? c.z : 0);
      }
    } else {
      for (int b = 0; b < nblk; ++b) {
        const int c = hq[b];
        t += c;
        if (b < me) pr += c;
      }
    }
    tot[u] = t;
    pre[u] = pr;
    mine += t;
  }
  int all;
  int off = block_excl_scan<256>(mine, tmp, &all);
#pragma unroll
  for (int u = 0; u < DPT; ++u) {
    const int q = tid * DPT + u;
    base[q] = off + pre[u];
    off += tot[u];
#pragma unroll
    for (int v = 0; v < 4; ++v) wcnt[v][q] = 0;
  }
  __syncthreads();
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int r = 0; r < RND; ++r) {
    const int i = blockIdx.x * kSortTile + r * 256 + tid;
    const bool valid = i < B;
    const int key = keys[r];
    const int val = vals[r];
    const uint32_t dig = (static_cast<uint32_t>(key) >> shift) & (NB - 1u);
    unsigned long long match = __ballot(valid);
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const bool bit = (dig >> b) & 1u;
      const unsigned long long bal = __ballot(bit);
      match &= bit ? bal : ~bal;
    }
    const int rank = __popcll(match & below);
    if (valid && rank == 0) wcnt[w][dig] = __popcll(match);
    __syncthreads();
    if (valid) {
      int pre = 0;
      for (int q = 0; q < w; ++q) pre += wcnt[q][dig];
      const int pos = base[dig] + pre + rank;
      kout[pos] = key;
      vout[pos] = val;
    }
    __syncthreads();
    for (int q = tid; q < NB; q += 256) {
      base[q] += wcnt[0][q] + wcnt[1][q] + wcnt[2][q] + wcnt[3][q];
#pragma unroll
      for (int v = 0; v < 4; ++v) wcnt[v][q] = 0;
    }
    __syncthreads();
  }
}

// Segment boundaries per 1024-token tile.
__global__ __launch_bounds__(256) void seg_count_kernel(const int32_t* sid,
                                                        int B, int32_t* blk) {
  __shared__ int tmp[256 / 64 + 1];
  const int tid = threadIdx.x;
  int c = 0;
  for (int r = 0; r < kSortTile / 256; ++r) {
    int j = blockIdx.x * kSortTile + r * 256 + tid;
    if (j < B && (j == 0 || sid[j] != sid[j - 1])) ++c;
  }
  int total;
  block_excl_scan<256>(c, tmp, &total);
  if (tid == 0) blk[blockIdx.x] = total;
}

// Write the segment arrays; blk holds the tiles' segment counts (each
// workgroup adds up those of the tiles before its own, and all of them: S).
// A thread's five ids and the rows of the ids that start a segment there
// are read before the counts, so the three reads overlap.
__global__ __launch_bounds__(256) void seg_write_kernel(PlanDev pd,
                                                        PlanParams p,
                                                        int nblk) {
  __shared__ int tmp[256 / 64 + 1];
  const int tid = threadIdx.x;
  const int B = p.B;
  // each thread takes 4 consecutive positions of the tile, in order; ids
  // of positions j0 - 1 .. j0 + 3
  const int j0 = blockIdx.x * kSortTile + tid * 4;
  int ids[5];
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    const int j = j0 - 1 + q;
    ids[q] = j >= 0 && j < B ? pd.sorted_ids[j] : 0;
  }
  bool head[4];
  int64_t r0[4];
  int n[4], c = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = j0 + q;
    head[q] = j < B && (j == 0 || ids[q + 1] != ids[q]);
    r0[q] = 0;
    n[q] = 0;
    if (head[q]) {
      id_rows(p, ids[q + 1], &r0[q], &n[q], pd.header);
      ++c;
    }
  }
  int before = 0, every = 0;
  for (int i = tid; i < nblk; i += 256) {
    const int cb = pd.blk[i];
    every += cb;
    if (i < static_cast<int>(blockIdx.x)) before += cb;
  }
  int first, S;
  block_excl_scan<256>(before, tmp, &first);
  block_excl_scan<256>(every, tmp, &S);
  int total;
  int s = first + block_excl_scan<256>(c, tmp, &total);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (head[q]) {
      pd.seg_id[s] = ids[q + 1];
      pd.seg_tok_start[s] = j0 + q;
      pd.seg_row_off[s] = r0[q];
      pd.seg_n[s] = n[q];
      ++s;
    }
  }
  if (blockIdx.x == 0 && tid == 0) {
    pd.seg_tok_start[S] = B;
    pd.header[1] = S;
  }
}

// Work items per segment, exclusive-scanned (a[S] = total); S is read on
// the device. One workgroup per count array, side by side: each first
// writes its segments' counts (coalesced, sixteen segments a thread), then scans
// them in place (the workgroup barrier orders its own global writes and
// reads): wave items (seg_item_start, header[2]), 64-token items
// (seg_gitem_start, header[3]), and with with_all the wave items of every
// id (seg_aitem_start, header[8]; without it header[8] repeats header[2]).
__global__ __launch_bounds__(1024) void seg_items_scan_kernel(PlanDev pd,
                                                              PlanParams p,
                                                              int with_all) {
  __shared__ int tmp[1024 / 64 + 1];
  const int n = pd.header[1];
  const int kind = blockIdx.x;
  int32_t* a = kind == 0   ? pd.seg_item_start
               : kind == 1 ? pd.seg_gitem_start
                           : pd.seg_aitem_start;
  for (int base = 0; base < n; base += 16 * 1024) {
    // sixteen segments a thread, every load of the round issued first
    int m[16], rows[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int g = min(base + k * 1024 + static_cast<int>(threadIdx.x), n - 1);
      m[k] = pd.seg_tok_start[g + 1] - pd.seg_tok_start[g];
      rows[k] = pd.seg_n[g];
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int g = base + k * 1024 + threadIdx.x;
      if (g < n)
        a[g] = kind == 0   ? items_of(m[k], rows[k], p)
               : kind == 1 ? gitems_of(m[k], rows[k], p)
                           : aitems_of(m[k], rows[k], p);
    }
  }
  __syncthreads();
  const int total = scan_excl_1024(a, n, tmp);
  if (threadIdx.x == 0) {
    a[n] = total;
    if (kind == 0) {
      pd.header[2] = total;
      if (!with_all) pd.header[8] = total;
    } else if (kind == 1) {
      pd.header[3] = total;
    } else {
      pd.header[8] = total;
    }
  }
}

// Direct maps from a work item to its segment and its index there, so the
// forward kernels need no search: one wavefront per segment writes the
// entries of all its items (its lanes side by side), whatever the kind;
// the 128-token items also go to a compact list of their own, all items of
// one id as one block of their XCD's list (reserved by one atomic; the
// order of the blocks depends on timing, the items' results do not).
__global__ __launch_bounds__(256) void item_map_kernel(PlanDev pd,
                                                       int with_all,
                                                       int64_t hcap) {
  if (pd.header[0] != 0) return;
  const int S = pd.header[1];
  const int lane = threadIdx.x & 63;
  const int waves = gridDim.x * 4;
  for (int g = blockIdx.x * 4 + (threadIdx.x >> 6); g < S; g += waves) {
    const int w0 = pd.seg_item_start[g], w1 = pd.seg_item_start[g + 1];
    const int q0 = pd.seg_gitem_start[g], q1 = pd.seg_gitem_start[g + 1];
    for (int i = w0 + lane; i < w1; i += 64)
      pd.item_map[i] = make_int2(g, i - w0);
    if (q1 > q0) {
      for (int i = q0 + lane; i < q1; i += 64)
        pd.gitem_map[i] = make_int2(g, i - q0);
      if (pd.seg_tok_start[g + 1] - pd.seg_tok_start[g] > kGroupTok) {
        const int x = hot_list_of(g);
        int first = 0;
        if (lane == 0) first = atomicAdd(&pd.header[16 + x], q1 - q0);
        first = __shfl(first, 0);
        int2* list = pd.hitem_map + x * hcap + first;
        for (int j = lane; j < q1 - q0; j += 64) list[j] = make_int2(g, j);
      }
    }
    if (with_all) {
      const int a0 = pd.seg_aitem_start[g], a1 = pd.seg_aitem_start[g + 1];
      for (int i = a0 + lane; i < a1; i += 64)
        pd.aitem_map[i] = make_int2(g, i - a0);
    }
  }
}

// one wavefront per segment, at most B segments
static int item_map_grid(int B) {
  const int g = ceil_div(B, 4);
  return g < 4096 ? (g > 0 ? g : 1) : 4096;
}

static int id_bits(int64_t vocab) {
  int bits = 1;
  while (bits < 32 && (int64_t(1) << bits) < vocab) ++bits;
  return bits;
}

hipError_t plan_launch(const PlanDev& pd, const PlanParams& p,
                       hipStream_t s) {
  const int B = p.B;
  if (B <= kTinyPlanMax && p.group_min_rows == 0) {
    plan_tiny_kernel<<<1, 64, 0, s>>>(pd, p);
    return hipGetLastError();
  }
  if (B <= kSmallPlanMax) {
    plan_small_kernel<<<1, 1024, 0, s>>>(pd, p);
    // (without group items the small plan writes the item map itself)
    if (p.group_min_rows > 0)
      item_map_kernel<<<item_map_grid(B), 256, 0, s>>>(pd, 1, hitem_cap(B));
    return hipGetLastError();
  }
  const int nblk = ceil_div(B, kSortTile);
  // 8-bit digits, or 9-bit ones where that saves a pass (17-18 bits and
  // 25-27 bits of id range)
  const int bits = id_bits(p.vocab);
  const int db = (bits + 8) / 9 < (bits + 7) / 8 ? 9 : 8;
  const int passes = (bits + db - 1) / db;
  // ping-pong so that the last pass lands in (sorted_ids, perm)
  int32_t* ka[2] = {pd.sorted_ids, pd.keys_alt};
  int32_t* va[2] = {pd.perm, pd.vals_alt};
  int out = (passes % 2 == 1) ? 0 : 1;
  const int32_t* kin = p.ids;
  const int32_t* vin = nullptr;
  for (int ps = 0; ps < passes; ++ps) {
    const int shift = db * ps;
    // pass 0: the id check's per-tile verdicts go to blk (rewritten by
    // seg_count later), and the scatter starts the header from them
    int32_t* bad = ps == 0 ? pd.blk : nullptr;
    int32_t* hdr = ps == 0 ? pd.header : nullptr;
    if (db == 9) {
      radix_hist_kernel<9><<<nblk, 256, 0, s>>>(kin, B, shift, pd.hist, nblk,
                                                p.vocab, bad);
      radix_scatter_kernel<9><<<nblk, 256, 0, s>>>(
          kin, vin, ka[out], va[out], B, shift, pd.hist, nblk, hdr, bad);
    } else {
      radix_hist_kernel<8><<<nblk, 256, 0, s>>>(kin, B, shift, pd.hist, nblk,
                                                p.vocab, bad);
      radix_scatter_kernel<8><<<nblk, 256, 0, s>>>(
          kin, vin, ka[out], va[out], B, shift, pd.hist, nblk, hdr, bad);
    }
    kin = ka[out];
    vin = va[out];
    out ^= 1;
  }
  seg_count_kernel<<<nblk, 256, 0, s>>>(pd.sorted_ids, B, pd.blk);
  seg_write_kernel<<<nblk, 256, 0, s>>>(pd, p, nblk);
  seg_items_scan_kernel<<<p.group_min_rows > 0 ? 3 : 2, 1024, 0, s>>>(
      pd, p, p.group_min_rows > 0);
  item_map_kernel<<<item_map_grid(B), 256, 0, s>>>(pd, p.group_min_rows > 0,
                                                  hitem_cap(B));
  return hipGetLastError();
}

}  // namespace l3
