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
// same permutation. Two implementations:
//   * batches up to 4096 tokens: one 1024-thread workgroup, bitonic sort of
//     64-bit keys in LDS, then segment cut and work-item count in the same
//     launch (one launch: decode-sized batches are latency bound);
//   * larger batches: LSD radix sort of the 32-bit ids with the position as
//     payload (stable, 8-bit digits, histogram / scan / ranked scatter per
//     digit), then segment cut kernels.
// After the segments, the plan counts the forward pass's work items: a
// segment with n_g >= group_min_rows (large batches only) yields
// ceil(m_g / 64) group items (seg_gitem_start), any other segment
// ceil(m_g / 32) * ceil(n_g / chunk) wave items (seg_item_start); both are
// exclusive prefix sums.

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

// ---------------------------------------------------------------- small ---
__global__ __launch_bounds__(1024) void plan_small_kernel(PlanDev pd,
                                                          PlanParams p) {
  __shared__ unsigned long long keys[kSmallPlanMax];
  __shared__ int tmp[1024 / 64 + 1];
  __shared__ int s_total;
  const int tid = threadIdx.x;
  const int B = p.B;
  int B2 = 1;
  while (B2 < B) B2 <<= 1;
  if (tid < 16) pd.header[tid] = 0;
  __syncthreads();

  for (int i = tid; i < B2; i += 1024) {
    unsigned long long k = ~0ull;
    if (i < B) {
      int t = p.ids[i];
      if (t < 0 || t >= p.vocab) atomicOr(&pd.header[0], kBadId);
      k = (static_cast<unsigned long long>(static_cast<uint32_t>(t)) << 32) |
          static_cast<uint32_t>(i);
    }
    keys[i] = k;
  }
  __syncthreads();
  // bitonic sort, ascending
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
      id_rows(p, t, &r0, &n, pd.header);
      pd.seg_id[s] = t;
      pd.seg_tok_start[s] = j;
      pd.seg_row_off[s] = r0;
      pd.seg_n[s] = n;
      ++s;
    }
  }
  if (tid == 0) {
    pd.seg_tok_start[S] = B;
    pd.header[1] = S;
  }
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
    pd.header[2] = total;
    pd.header[3] = gtotal;
    pd.header[8] = atotal;
  }
  (void)s_total;
}

// ---------------------------------------------------------------- large ---
__global__ void header_init_kernel(int32_t* header) {
  if (threadIdx.x < 16) header[threadIdx.x] = 0;
}

// Digit histogram of one 1024-key tile (DB-bit digits, 2^DB buckets);
// pass 0 also checks the id range.
template <int DB>
__global__ __launch_bounds__(256) void radix_hist_kernel(
    const int32_t* kin, int B, int shift, int32_t* hist, int nblk,
    int64_t vocab, int32_t* header, int validate) {
  constexpr int NB = 1 << DB;
  __shared__ int h[NB];
  const int tid = threadIdx.x;
  for (int q = tid; q < NB; q += 256) h[q] = 0;
  __syncthreads();
  for (int r = 0; r < kSortTile / 256; ++r) {
    int i = blockIdx.x * kSortTile + r * 256 + tid;
    if (i < B) {
      int k = kin[i];
      if (validate && (k < 0 || k >= vocab)) atomicOr(&header[0], kBadId);
      atomicAdd(&h[(static_cast<uint32_t>(k) >> shift) & (NB - 1u)], 1);
    }
  }
  __syncthreads();
  for (int q = tid; q < NB; q += 256) hist[q * nblk + blockIdx.x] = h[q];
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

// In-place exclusive scan of n ints; the total goes to *total_out when given.
__global__ __launch_bounds__(1024) void scan_single_kernel(int32_t* a, int n,
                                                           int32_t* total_out) {
  __shared__ int tmp[1024 / 64 + 1];
  const int total = scan_excl_1024(a, n, tmp);
  if (threadIdx.x == 0 && total_out) *total_out = total;
}

// Stable scatter of one 1024-key tile by one DB-bit digit. Keys of a tile
// are taken in order, 256 at a time; within a wave the rank among equal
// digits comes from a ballot match on the digit bits, across waves from LDS
// counts.
template <int DB>
__global__ __launch_bounds__(256) void radix_scatter_kernel(
    const int32_t* kin, const int32_t* vin, int32_t* kout, int32_t* vout,
    int B, int shift, const int32_t* hist, int nblk) {
  constexpr int NB = 1 << DB;
  __shared__ int base[NB];
  __shared__ int wcnt[4][NB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int q = tid; q < NB; q += 256) {
    base[q] = hist[q * nblk + blockIdx.x];
#pragma unroll
    for (int v = 0; v < 4; ++v) wcnt[v][q] = 0;
  }
  __syncthreads();
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int r = 0; r < kSortTile / 256; ++r) {
    const int i = blockIdx.x * kSortTile + r * 256 + tid;
    const bool valid = i < B;
    const int key = valid ? kin[i] : 0;
    const int val = valid ? (vin ? vin[i] : i) : 0;
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

// Write the segment arrays; blk holds the exclusive scan of the tile counts
// and blk[nblk] the total S.
__global__ __launch_bounds__(256) void seg_write_kernel(PlanDev pd,
                                                        PlanParams p,
                                                        int nblk) {
  __shared__ int tmp[256 / 64 + 1];
  const int tid = threadIdx.x;
  const int B = p.B;
  // each thread takes 4 consecutive positions of the tile, in order
  const int j0 = blockIdx.x * kSortTile + tid * 4;
  int c = 0;
  for (int q = 0; q < 4; ++q) {
    int j = j0 + q;
    if (j < B && (j == 0 || pd.sorted_ids[j] != pd.sorted_ids[j - 1])) ++c;
  }
  int total;
  int s = pd.blk[blockIdx.x] + block_excl_scan<256>(c, tmp, &total);
  for (int q = 0; q < 4; ++q) {
    int j = j0 + q;
    if (j < B && (j == 0 || pd.sorted_ids[j] != pd.sorted_ids[j - 1])) {
      int t = pd.sorted_ids[j];
      int64_t r0;
      int n;
      id_rows(p, t, &r0, &n, pd.header);
      pd.seg_id[s] = t;
      pd.seg_tok_start[s] = j;
      pd.seg_row_off[s] = r0;
      pd.seg_n[s] = n;
      ++s;
    }
  }
  if (blockIdx.x == 0 && tid == 0) {
    const int S = pd.blk[nblk];
    pd.seg_tok_start[S] = B;
    pd.header[1] = S;
  }
}

// Work items per segment (into seg_item_start / seg_gitem_start, scanned
// afterwards).
__global__ __launch_bounds__(256) void seg_items_kernel(PlanDev pd,
                                                        PlanParams p) {
  const int S = pd.header[1];
  for (int g = blockIdx.x * 256 + threadIdx.x; g < S;
       g += gridDim.x * 256) {
    const int m = pd.seg_tok_start[g + 1] - pd.seg_tok_start[g];
    pd.seg_item_start[g] = items_of(m, pd.seg_n[g], p);
    pd.seg_gitem_start[g] = gitems_of(m, pd.seg_n[g], p);
    if (p.group_min_rows > 0)
      pd.seg_aitem_start[g] = aitems_of(m, pd.seg_n[g], p);
  }
}

// Scan the item counts in place (a[S] = total); S is read on the device.
// One workgroup per count array, side by side: wave items (header[2]),
// 64-token items (header[3]), and with with_all the wave items of every id
// (header[8]; without it header[8] repeats header[2]).
__global__ __launch_bounds__(1024) void seg_items_scan_kernel(PlanDev pd,
                                                              int with_all) {
  __shared__ int tmp[1024 / 64 + 1];
  const int n = pd.header[1];
  int32_t* a = blockIdx.x == 0   ? pd.seg_item_start
               : blockIdx.x == 1 ? pd.seg_gitem_start
                                 : pd.seg_aitem_start;
  const int total = scan_excl_1024(a, n, tmp);
  if (threadIdx.x == 0) {
    a[n] = total;
    if (blockIdx.x == 0) {
      pd.header[2] = total;
      if (!with_all) pd.header[8] = total;
    } else if (blockIdx.x == 1) {
      pd.header[3] = total;
    } else {
      pd.header[8] = total;
    }
  }
}

// Direct maps from a work item to its segment and its index there, so the
// forward kernels need no search: one thread per item finds its segment by
// binary search over the segments' first items (parallel over items, so a
// segment with thousands of items costs no more than one with one).
__device__ __forceinline__ int seg_of(const int32_t* start, int S, int i) {
  int lo = 0, hi = S - 1;  // last g with start[g] <= i
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (start[mid] <= i)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void item_map_kernel(PlanDev pd,
                                                       int with_all) {
  if (pd.header[0] != 0) return;
  const int S = pd.header[1];
  const int n_wave = pd.header[2], n_group = pd.header[3];
  const int n_all = with_all ? pd.header[8] : 0;
  const int n = max(n_wave, max(n_group, n_all));
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
    if (i < n_wave) {
      const int g = seg_of(pd.seg_item_start, S, i);
      pd.item_map[i] = make_int2(g, i - pd.seg_item_start[g]);
    }
    if (i < n_group) {
      const int g = seg_of(pd.seg_gitem_start, S, i);
      const int j = i - pd.seg_gitem_start[g];
      pd.gitem_map[i] = make_int2(g, j);
      // the 128-token items also go to a compact list of their own (its
      // order depends on timing; the items' results do not)
      if (pd.seg_tok_start[g + 1] - pd.seg_tok_start[g] > kGroupTok)
        pd.hitem_map[atomicAdd(&pd.header[6], 1)] = make_int2(g, j);
    }
    if (i < n_all) {
      const int g = seg_of(pd.seg_aitem_start, S, i);
      pd.aitem_map[i] = make_int2(g, i - pd.seg_aitem_start[g]);
    }
  }
}

static int item_map_grid(int B) {
  const int64_t cap = wave_items_cap(B);
  const int64_t g = (cap + 255) / 256;
  return static_cast<int>(g < 2048 ? (g > 0 ? g : 1) : 2048);
}

static int id_bits(int64_t vocab) {
  int bits = 1;
  while (bits < 32 && (int64_t(1) << bits) < vocab) ++bits;
  return bits;
}

hipError_t plan_launch(const PlanDev& pd, const PlanParams& p,
                       hipStream_t s) {
  const int B = p.B;
  if (B <= kSmallPlanMax) {
    plan_small_kernel<<<1, 1024, 0, s>>>(pd, p);
    item_map_kernel<<<item_map_grid(B), 256, 0, s>>>(pd, p.group_min_rows > 0);
    return hipGetLastError();
  }
  const int nblk = ceil_div(B, kSortTile);
  header_init_kernel<<<1, 64, 0, s>>>(pd.header);
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
    if (db == 9) {
      radix_hist_kernel<9><<<nblk, 256, 0, s>>>(kin, B, shift, pd.hist, nblk,
                                                p.vocab, pd.header, ps == 0);
      scan_single_kernel<<<1, 1024, 0, s>>>(pd.hist, 512 * nblk, nullptr);
      radix_scatter_kernel<9><<<nblk, 256, 0, s>>>(
          kin, vin, ka[out], va[out], B, shift, pd.hist, nblk);
    } else {
      radix_hist_kernel<8><<<nblk, 256, 0, s>>>(kin, B, shift, pd.hist, nblk,
                                                p.vocab, pd.header, ps == 0);
      scan_single_kernel<<<1, 1024, 0, s>>>(pd.hist, 256 * nblk, nullptr);
      radix_scatter_kernel<8><<<nblk, 256, 0, s>>>(
          kin, vin, ka[out], va[out], B, shift, pd.hist, nblk);
    }
    kin = ka[out];
    vin = va[out];
    out ^= 1;
  }
  seg_count_kernel<<<nblk, 256, 0, s>>>(pd.sorted_ids, B, pd.blk);
  scan_single_kernel<<<1, 1024, 0, s>>>(pd.blk, nblk, pd.blk + nblk);
  seg_write_kernel<<<nblk, 256, 0, s>>>(pd, p, nblk);
  seg_items_kernel<<<ceil_div(B, 256), 256, 0, s>>>(pd, p);
  seg_items_scan_kernel<<<p.group_min_rows > 0 ? 3 : 2, 1024, 0, s>>>(
      pd, p.group_min_rows > 0);
  item_map_kernel<<<item_map_grid(B), 256, 0, s>>>(pd, p.group_min_rows > 0);
  return hipGetLastError();
}

}  // namespace l3
