// Segment forward, wave kernel: a_i = V_t^T Softmax(K_t x_i) for every
// token, one wave item (segment, tile of <= 16 of its tokens, chunk of
// <= 128 of its rows; seg_wave.h) per wavefront. It serves everything the
// one-launch group kernel does not: float32 inputs, batches of up to 2048
// tokens, and the saving forward of training (float32 weights). Four
// independent wavefronts a workgroup (no workgroup barrier), items taken
// round-robin, two workgroups a CU.
//
// gist.science explainer of "L^3: Large Lookup Layers", Technical Summary,
// Core Architecture: after the static lookup of K_t and V_t, the hidden
// state attends over them (Context-Dependent Aggregation), giving
// V_t^T Softmax(K_t x) inside the Mathematical Formulation. Systems-Friendly
// Design, Batch Sorting: grouping tokens by id makes the mask
// block-diagonal, so one block of tokens shares one read of K_t, V_t.
//
// Ids whose rows span several chunks leave (max, sum, acc) partials per
// chunk; seg_combine_kernel merges them per token in chunk order (exact,
// deterministic).

#include "seg_wave.h"

namespace l3 {

// Most row chunks of one id: k_max <= 512 rows in chunks of >= 32.
constexpr int kMaxChunks = 16;

template <bool BF16, int EPL, bool P32>
__global__ __launch_bounds__(256, 2) void seg_fwd_kernel(SegFwdArgs a) {
  typedef typename Types<BF16, P32>::P PT;
  __shared__ PT s_p[4][kNBMax * 16 * kTokTile];
  __shared__ float s_ml[4][2 * kTokTile];
  if (a.header[0] != 0) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n_items = a.header[a.count_slot];
  const int G = gridDim.x;
  // With fewer items than wavefronts (small batches) the items go to the
  // first wave of every workgroup before the second, so that they spread
  // over all CUs; otherwise consecutive items share a workgroup. Either
  // order visits every item once.
  const bool spread = n_items < G * 4;
  for (int item = spread ? blockIdx.x + w * G : blockIdx.x * 4 + w;
       item < n_items; item += G * 4)
    wave_item<BF16, EPL, P32>(a, item, lane, s_p[w], s_ml[w]);
}

// Merge the row-chunk partials of every token whose id needed more than one
// chunk: M = max_c m_c, L = sum_c l_c e^(m_c - M),
// a = sum_c acc_c e^(m_c - M) / L, chunks taken in order.
template <bool BF16>
__global__ __launch_bounds__(256) void seg_combine_kernel(CombineArgs a) {
  typedef typename Types<BF16>::T T;
  if (a.header[0] != 0) return;
  const int lane = threadIdx.x & 63;
  const int pos = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pos >= a.B) return;
  const int S = a.header[1];
  // The token's segment, the last s with seg_tok_start[s] <= pos (starts
  // ascend strictly), by a 64-ary search: each round the wave's lanes test
  // 64 evenly spaced candidates in [lo, hi] at once and keep the span after
  // the last one that passes (lane 0's candidate lo always does), so up to
  // 64 segments take one round of loads and 65536 take three.
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int step = (hi - lo + 64) / 64;
    const int c = lo + lane * step;
    const bool ok = c <= hi && a.seg_tok_start[c] <= pos;
    const int k = __popcll(__ballot(ok));
    lo += (k - 1) * step;
    hi = min(hi, lo + step - 1);
  }
  const int n_rows = a.seg_n[lo];
  if (a.group_min_rows > 0 && n_rows >= a.group_min_rows) return;
  const int nch = ceil_div(n_rows, a.chunk_rows);
  if (nch <= 1) return;
  const int64_t slot0 = static_cast<int64_t>(pos) * a.nch_max;
  // chunk weights w_c = e^(m_c - M) / L, all chunks' loads issued together;
  // with d_e <= 512 the chunks' partial rows (four columns a lane in each
  // 256-column block) are loaded in the same burst, before the weights
  // are known (chunks past nch and columns past d_e re-read chunk 0 /
  // column 0, inside the buffer, and are never used)
  float m[kMaxChunks], l[kMaxChunks], w[kMaxChunks];
  constexpr int kPB = 2;
  const bool pre = a.d_e <= kPB * 256;
  float4 pv[kMaxChunks][kPB];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int cc = c < nch ? c : 0;
    const float2 v =
        *reinterpret_cast<const float2*>(a.part_ml + (slot0 + cc) * 2);
    m[c] = c < nch ? v.x : -INFINITY;
    l[c] = c < nch ? v.y : 0.f;
    if (pre) {
#pragma unroll
      for (int b = 0; b < kPB; ++b) {
        const int e = b * 256 + lane * 4;
        pv[c][b] = *reinterpret_cast<const float4*>(
            a.part + (slot0 + cc) * a.d_e + (e < a.d_e ? e : 0));
      }
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) M = fmaxf(M, m[c]);
  float L = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    w[c] = c < nch ? __expf(m[c] - M) : 0.f;
    L += l[c] * w[c];
  }
  const float invL = 1.0f / L;
  const int64_t orig = a.perm[pos];
  auto emit = [&](int e, const float4& acc) __attribute__((always_inline)) {
    const float o[4] = {acc.x * invL, acc.y * invL, acc.z * invL,
                        acc.w * invL};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      st<T>(static_cast<T*>(a.a_out), orig * a.d_e + e + q, o[q]);
      if (a.a_save) a.a_save[orig * a.d_e + e + q] = o[q];
    }
  };
  if (pre) {
#pragma unroll
    for (int b = 0; b < kPB; ++b) {
      const int e = b * 256 + lane * 4;
      if (e < a.d_e) {
        float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) {
          if (c < nch) {
            acc.x = fmaf(pv[c][b].x, w[c], acc.x);
            acc.y = fmaf(pv[c][b].y, w[c], acc.y);
            acc.z = fmaf(pv[c][b].z, w[c], acc.z);
            acc.w = fmaf(pv[c][b].w, w[c], acc.w);
          }
        }
        emit(e, acc);
      }
    }
    return;
  }
  // 4 columns a lane, the chunks' partial rows loaded together
  for (int e = lane * 4; e < a.d_e; e += 256) {
    float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      if (c < nch) {
        const float4 v = *reinterpret_cast<const float4*>(
            a.part + (slot0 + c) * a.d_e + e);
        acc.x = fmaf(v.x, w[c], acc.x);
        acc.y = fmaf(v.y, w[c], acc.y);
        acc.z = fmaf(v.z, w[c], acc.z);
        acc.w = fmaf(v.w, w[c], acc.w);
      }
    }
    emit(e, acc);
  }
}

template <bool BF16, bool P32>
static hipError_t seg_fwd_dispatch(const SegFwdArgs& a, int grid,
                                   hipStream_t s) {
  // EPL: value columns per lane per pass (at most 4, the rest in passes)
  const int q = a.d_e / 64;  // d_e is a multiple of 64
  const int epl = q % 4 == 0 ? 4 : q % 2 == 0 ? 2 : 1;
  switch (epl) {
    case 4:
      seg_fwd_kernel<BF16, 4, P32><<<grid, 256, 0, s>>>(a);
      break;
    case 2:
      seg_fwd_kernel<BF16, 2, P32><<<grid, 256, 0, s>>>(a);
      break;
    default:
      seg_fwd_kernel<BF16, 1, P32><<<grid, 256, 0, s>>>(a);
      break;
  }
  return hipGetLastError();
}

hipError_t seg_fwd_launch(const SegFwdArgs& a, int dtype, int B, int items_ub,
                          hipStream_t s) {
  (void)B;
  int grid = ceil_div(items_ub, 4);
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  if (dtype != kBF16) return seg_fwd_dispatch<false, true>(a, grid, s);
  // float32 weights when the aggregate is saved for the backward pass
  return a.a_save ? seg_fwd_dispatch<true, true>(a, grid, s)
                  : seg_fwd_dispatch<true, false>(a, grid, s);
}

hipError_t seg_combine_launch(const CombineArgs& a, int dtype,
                              hipStream_t s) {
  const int grid = ceil_div(a.B, 4);
  if (dtype == kBF16)
    seg_combine_kernel<true><<<grid, 256, 0, s>>>(a);
  else
    seg_combine_kernel<false><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace l3
