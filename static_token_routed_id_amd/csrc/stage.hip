// Staging of the batch's table rows from host memory into HBM.
//
// gist.science explainer of "L^3: Large Lookup Layers", Technical Summary,
// Systems-Friendly Design: the tables can live in CPU memory, because the
// rows a token needs follow from its id alone (Core Architecture, Static
// Routing) and can be fetched before the layer runs. Here the plan's
// segments say which rows: every id of the batch owns one contiguous slice
// of K and of V, so staging is one contiguous copy per id into compact
// device tables, after which the plan's row offsets point into them.
//
// Two kernels, both stream-ordered after the plan:
//   stage_offsets_kernel  one workgroup: exclusive prefix sum of the
//                         segments' row counts (the compact offsets); if the
//                         total exceeds the staging capacity the plan's
//                         status word gets kBadStage and every later kernel
//                         of the plan does nothing;
//   stage_copy_kernel     a few workgroups, one segment each at a time:
//                         copies the id's K and V rows (contiguous on both
//                         sides, read across the host link in 16-byte
//                         pieces, eight a thread in flight), then points the
//                         segment at its copy.

#include "l3_device.h"
#include "l3_internal.h"

namespace l3 {

#ifndef L3_STAGE_WGS
#define L3_STAGE_WGS 16
#endif
constexpr int kStageWGs = L3_STAGE_WGS;

__global__ __launch_bounds__(1024) void stage_offsets_kernel(StageArgs a) {
  __shared__ int64_t s_part[1024];
  if (a.header[0] != 0) return;
  const int S = a.header[1];
  const int tid = threadIdx.x;
  // thread t sums segments [t * per, (t + 1) * per)
  const int per = (S + 1023) / 1024;
  const int s0 = tid * per, s1 = min(S, s0 + per);
  int64_t sum = 0;
  for (int s = s0; s < s1; ++s) sum += a.seg_n[s];
  s_part[tid] = sum;
  __syncthreads();
  // inclusive scan of the 1024 partial sums (Hillis-Steele)
  for (int o = 1; o < 1024; o <<= 1) {
    const int64_t v = tid >= o ? s_part[tid - o] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  int64_t off = tid > 0 ? s_part[tid - 1] : 0;
  for (int s = s0; s < s1; ++s) {
    a.stage_off[s] = off;
    off += a.seg_n[s];
  }
  if (tid == 1023 && s_part[1023] > a.stage_rows)
    atomicOr(&a.header[0], kBadStage);
}

__global__ __launch_bounds__(256) void stage_copy_kernel(StageArgs a) {
  if (a.header[0] != 0) return;
  const int S = a.header[1];
  const int tid = threadIdx.x;
  const int64_t kb = static_cast<int64_t>(a.d) * a.elem;     // bytes a K row
  const int64_t vb = static_cast<int64_t>(a.d_e) * a.elem;   // bytes a V row
  for (int s = blockIdx.x; s < S; s += gridDim.x) {
    const int64_t src = a.seg_row_off[s];
    const int64_t dst = a.stage_off[s];
    const int64_t n = a.seg_n[s];
    // K then V: contiguous byte ranges, 16 bytes a thread, four in flight
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t rb = t == 0 ? kb : vb;
      const u32x4* from = reinterpret_cast<const u32x4*>(
          (t == 0 ? a.K_host : a.V_host) + src * rb);
      u32x4* to = reinterpret_cast<u32x4*>((t == 0 ? a.K_stage : a.V_stage) +
                                           dst * rb);
      const int64_t q = n * rb / 16;
      int64_t i = tid;
      for (; i + 7 * 256 < q; i += 8 * 256) {
        u32x4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = from[i + k * 256];
#pragma unroll
        for (int k = 0; k < 8; ++k) to[i + k * 256] = v[k];
      }
      for (; i < q; i += 256) to[i] = from[i];
    }
    // every thread has read this segment's source offset
    __syncthreads();
    if (tid == 0) a.seg_row_off[s] = dst;
  }
}

hipError_t stage_rows_launch(const StageArgs& a, int S_ub, hipStream_t s) {
  if (S_ub <= 0) return hipSuccess;
  stage_offsets_kernel<<<1, 1024, 0, s>>>(a);
  // few workgroups (each with 32 KB of reads in flight): the host link,
  // not the CUs, bounds the copy, and the CUs stay free for the layers the
  // copy is meant to overlap
  const int grid = S_ub < kStageWGs ? S_ub : kStageWGs;
  stage_copy_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace l3
