// Backward pass of the layer (the chain rule of the forward formula of the
// gist.science explainer of "L^3: Large Lookup Layers", Technical Summary,
// Core Architecture, Mathematical Formulation; the pages print no
// gradients). The projections' gradients run through gemm_generic; this
// file holds the LayerNorm backward and the per-id segment backward.
//
// Determinism: nothing here uses floating-point atomics. LayerNorm column
// sums (dgamma, dbeta) are taken by one thread per column over the rows in
// order. The segment backward gives each id (segment) to one workgroup,
// which walks that id's tokens in sorted order and is the only writer of the
// id's dK / dV rows (Systems-Friendly Design, Batch Sorting: the sorted
// batch makes the mask block-diagonal, so ids never share rows).

#include "l3_device.h"
#include "l3_internal.h"

namespace l3 {

__global__ __launch_bounds__(256) void fill_zero_kernel(float* p, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
       i < n; i += stride)
    p[i] = 0.f;
}

hipError_t fill_zero_launch(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  fill_zero_kernel<<<static_cast<int>(blocks), 256, 0, s>>>(p, n);
  return hipGetLastError();
}

// du = rstd * (g - mean(g) - uhat * mean(g * uhat)), g = gamma * dh.
template <typename T>
__global__ __launch_bounds__(256) void ln_bwd_rows_kernel(BwdArgs a) {
  if (a.header[0] != 0) return;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.B) return;
  const T* gamma = static_cast<const T*>(a.gamma);
  const int64_t base = static_cast<int64_t>(row) * a.d;
  float sg = 0.f, sgu = 0.f;
  for (int e = lane; e < a.d; e += 64) {
    const float gv = ld<T>(gamma, e) * a.dH[base + e];
    sg += gv;
    sgu += gv * a.uhat[base + e];
  }
  const float mg = wave_sum(sg) / a.d;
  const float mgu = wave_sum(sgu) / a.d;
  const float rstd = a.rstd[row];
  for (int e = lane; e < a.d; e += 64) {
    const float gv = ld<T>(gamma, e) * a.dH[base + e];
    a.dU[base + e] = rstd * (gv - mg - a.uhat[base + e] * mgu);
  }
}

// dgamma[j] = sum_i dh[i, j] * uhat[i, j], dbeta[j] = sum_i dh[i, j].
__global__ __launch_bounds__(256) void ln_bwd_cols_kernel(BwdArgs a) {
  if (a.header[0] != 0) return;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= a.d) return;
  float sg = 0.f, sb = 0.f;
  for (int i = 0; i < a.B; ++i) {
    const int64_t o = static_cast<int64_t>(i) * a.d + j;
    sg += a.dH[o] * a.uhat[o];
    sb += a.dH[o];
  }
  a.dgamma[j] = sg;
  a.dbeta[j] = sb;
}

hipError_t ln_bwd_launch(const BwdArgs& a, int dtype, hipStream_t s) {
  if (a.B > 0) {
    if (dtype == kBF16)
      ln_bwd_rows_kernel<uint16_t><<<ceil_div(a.B, 4), 256, 0, s>>>(a);
    else
      ln_bwd_rows_kernel<float><<<ceil_div(a.B, 4), 256, 0, s>>>(a);
  }
  ln_bwd_cols_kernel<<<ceil_div(a.d, 256), 256, 0, s>>>(a);
  return hipGetLastError();
}

// Fixed-order reduction over the 256 threads of a workgroup.
__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = is_max ? wave_max(v) : wave_sum(v);
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int q = 1; q < 4; ++q) r = is_max ? fmaxf(r, red[q]) : r + red[q];
  __syncthreads();
  return r;
}

// One workgroup per id. For each of the id's tokens i in sorted order:
// recompute p = Softmax(K_t x_i), dp = V_t da_i, ds = p * (dp - p . dp);
// dV_t += p da_i^T, dK_t += ds x_i^T (this workgroup owns those rows);
// dx_i += K_t^T ds.
template <typename T>
__global__ __launch_bounds__(256) void seg_bwd_kernel(BwdArgs a) {
  __shared__ float xs[4096];
  __shared__ float das[4096];
  __shared__ float ps[L3_MAX_ROWS_PER_ID];
  __shared__ float dss[L3_MAX_ROWS_PER_ID];
  __shared__ float red[4];
  if (a.header[0] != 0) return;
  const int S = a.header[1];
  const int tid = threadIdx.x;
  const T* X = static_cast<const T*>(a.x);
  const T* K = static_cast<const T*>(a.K);
  const T* V = static_cast<const T*>(a.V);
  for (int s = blockIdx.x; s < S; s += gridDim.x) {
    const int t0 = a.seg_tok_start[s], t1 = a.seg_tok_start[s + 1];
    const int n = a.seg_n[s];
    const int64_t r0 = a.seg_row_off[s];
    for (int tk = t0; tk < t1; ++tk) {
      const int64_t i = a.perm[tk];
      for (int c = tid; c < a.d; c += 256) xs[c] = ld<T>(X, i * a.d + c);
      for (int c = tid; c < a.d_e; c += 256) das[c] = a.dA[i * a.d_e + c];
      __syncthreads();
      float mx = -INFINITY;
      for (int j = tid; j < n; j += 256) {
        const int64_t rk = (r0 + j) * a.d, rv = (r0 + j) * a.d_e;
        float sc = 0.f, dp = 0.f;
        for (int c = 0; c < a.d; ++c) sc = fmaf(ld<T>(K, rk + c), xs[c], sc);
        for (int c = 0; c < a.d_e; ++c) dp = fmaf(ld<T>(V, rv + c), das[c], dp);
        ps[j] = sc;
        dss[j] = dp;
        mx = fmaxf(mx, sc);
      }
      mx = block_reduce(mx, red, true);
      float sum = 0.f;
      for (int j = tid; j < n; j += 256) {
        const float e = __expf(ps[j] - mx);
        ps[j] = e;
        sum += e;
      }
      sum = block_reduce(sum, red, false);
      const float inv = 1.0f / sum;
      float pdp = 0.f;
      for (int j = tid; j < n; j += 256) {
        const float p = ps[j] * inv;
        ps[j] = p;
        pdp = fmaf(p, dss[j], pdp);
      }
      pdp = block_reduce(pdp, red, false);
      for (int j = tid; j < n; j += 256) dss[j] = ps[j] * (dss[j] - pdp);
      __syncthreads();
      for (int idx = tid; idx < n * a.d_e; idx += 256) {
        const int j = idx / a.d_e, c = idx - j * a.d_e;
        a.dV[(r0 + j) * a.d_e + c] += ps[j] * das[c];
      }
      for (int idx = tid; idx < n * a.d; idx += 256) {
        const int j = idx / a.d, c = idx - j * a.d;
        a.dK[(r0 + j) * a.d + c] += dss[j] * xs[c];
      }
      for (int c = tid; c < a.d; c += 256) {
        float acc = 0.f;
        for (int j = 0; j < n; ++j)
          acc = fmaf(dss[j], ld<T>(K, (r0 + j) * a.d + c), acc);
        a.dx[i * a.d + c] += acc;
      }
      __syncthreads();
    }
  }
}

hipError_t seg_bwd_launch(const BwdArgs& a, int dtype, int S_ub,
                          hipStream_t s) {
  if (S_ub <= 0) return hipSuccess;
  const int grid = S_ub < 4096 ? S_ub : 4096;
  if (dtype == kBF16)
    seg_bwd_kernel<uint16_t><<<grid, 256, 0, s>>>(a);
  else
    seg_bwd_kernel<float><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace l3
