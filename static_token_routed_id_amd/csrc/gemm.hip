// Dense parts of the layer: the W_up and W_mix projections and LayerNorm
// (gist.science explainer of "L^3: Large Lookup Layers", Technical Summary,
// Core Architecture, Mathematical Formulation:
// y = W_mix [LayerNorm(W_up a) ; x] with a = V_t^T Softmax(K_t x)).
//
// * gemm_nt_mfma: bf16 inputs, f32 accumulation on 16x16x32 MFMA. Both
//   operands are K-contiguous ("NT": C = A B^T with A [M x K], B [N x K]),
//   which is the layout of every forward projection: u = a W_up^T and
//   y = [h ; x] W_mix^T. The A operand switches from its first to its
//   second source at column K1, so W_mix [W_a | W_b] multiplies h and x
//   without building the concatenation. Tile 128 x 128 x 64, four waves
//   each owning 64 x 64 (4 x 4 MFMA blocks); tiles are staged through LDS
//   with rows padded to 72 elements (16 lanes reading one 16-byte slice of
//   16 rows then hit 64 distinct banks) and the next K slice is prefetched
//   into registers while the current one is multiplied.
// * gemm_generic: float32 FMA with arbitrary strides and element types,
//   used for small shapes, float32 inputs and the backward pass.
// * layernorm_rows: one wave per row, two-pass mean / biased variance.

#include "l3_device.h"
#include "l3_internal.h"

namespace l3 {

// ---------------------------------------------------------------- generic ---
template <typename TA, typename TB, typename TC>
__global__ __launch_bounds__(256) void gemm_generic_kernel(GemmArgs g) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  if (g.header && g.header[0] != 0) return;
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tm = tid >> 4, tn = tid & 15;
  const TA* A1 = static_cast<const TA*>(g.A1);
  const TA* A2 = static_cast<const TA*>(g.A2);
  const TB* Bm = static_cast<const TB*>(g.Bm);
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < g.K; k0 += 16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + q * 256;
      const int kk = e >> 6, mm = e & 63;
      const int gm = m0 + mm, gk = k0 + kk;
      float v = 0.f;
      if (gm < g.M && gk < g.K) {
        v = gk < g.K1 ? ld<TA>(A1, gm * g.a1_m + gk * g.a1_k)
                      : ld<TA>(A2, gm * g.a2_m + (gk - g.K1) * g.a2_k);
      }
      As[kk][mm] = v;
      const int gn = n0 + mm;
      float b = 0.f;
      if (gn < g.N && gk < g.K) b = ld<TB>(Bm, gk * g.b_k + gn * g.b_n);
      Bs[kk][mm] = b;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][tm * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tn * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  TC* C = static_cast<TC*>(g.C);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gm = m0 + tm * 4 + i;
    if (gm >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tn * 4 + j;
      if (gn < g.N) st<TC>(C, gm * g.c_m + gn, acc[i][j]);
    }
  }
}

template <typename TA, typename TB>
static void gemm_generic_c(const GemmArgs& g, int c_type, dim3 grid,
                           hipStream_t s) {
  if (c_type == kBF16)
    gemm_generic_kernel<TA, TB, uint16_t><<<grid, 256, 0, s>>>(g);
  else
    gemm_generic_kernel<TA, TB, float><<<grid, 256, 0, s>>>(g);
}

hipError_t gemm_launch(const GemmArgs& g, int a_type, int b_type, int c_type,
                       hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  dim3 grid(ceil_div(g.N, 64), ceil_div(g.M, 64));
  if (a_type == kBF16) {
    if (b_type == kBF16)
      gemm_generic_c<uint16_t, uint16_t>(g, c_type, grid, s);
    else
      gemm_generic_c<uint16_t, float>(g, c_type, grid, s);
  } else {
    if (b_type == kBF16)
      gemm_generic_c<float, uint16_t>(g, c_type, grid, s);
    else
      gemm_generic_c<float, float>(g, c_type, grid, s);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------- bf16 MFMA ---
constexpr int kBM = 128, kBN = 128, kBK = 64, kLDK = kBK + 8;

template <typename TC>
__global__ __launch_bounds__(256) void gemm_nt_mfma_kernel(GemmArgs g) {
  __shared__ uint16_t As[kBM * kLDK];
  __shared__ uint16_t Bs[kBN * kLDK];
  if (g.header && g.header[0] != 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int m0 = blockIdx.y * kBM, n0 = blockIdx.x * kBN;
  const uint16_t* A1 = static_cast<const uint16_t*>(g.A1);
  const uint16_t* A2 = static_cast<const uint16_t*>(g.A2);
  const uint16_t* Bm = static_cast<const uint16_t*>(g.Bm);
  // global -> LDS mapping: 8 threads per 128-byte row slice, 32 rows a pass
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  int64_t arow[4], brow[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    arow[q] = min(m0 + lr + 32 * q, g.M - 1);
    brow[q] = min(n0 + lr + 32 * q, g.N - 1);
  }
  uint4 ra[4], rb[4];
  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint16_t* src =
          k0 < g.K1 ? A1 + arow[q] * g.a1_m + k0 + lc
                    : A2 + arow[q] * g.a2_m + (k0 - g.K1) + lc;
      ra[q] = *reinterpret_cast<const uint4*>(src);
      rb[q] = *reinterpret_cast<const uint4*>(Bm + brow[q] * g.b_n + k0 + lc);
    }
  };
  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int r = lane & 15, kg = (lane >> 4) * 8;
  load_tiles(0);
  for (int k0 = 0; k0 < g.K; k0 += kBK) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<uint4*>(&As[(lr + 32 * q) * kLDK + lc]) = ra[q];
      *reinterpret_cast<uint4*>(&Bs[(lr + 32 * q) * kLDK + lc]) = rb[q];
    }
    __syncthreads();
    if (k0 + kBK < g.K) load_tiles(k0 + kBK);
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      uint4 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const uint4*>(
            &As[(wm * 64 + i * 16 + r) * kLDK + kk + kg]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const uint4*>(
            &Bs[(wn * 64 + j * 16 + r) * kLDK + kk + kg]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(af[i], bf[j], acc[i][j]);
    }
  }
  TC* C = static_cast<TC*>(g.C);
  const int g4 = (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int gm = m0 + wm * 64 + i * 16 + g4 + q;
      if (gm >= g.M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int gn = n0 + wn * 64 + j * 16 + r;
        st<TC>(C, static_cast<int64_t>(gm) * g.c_m + gn, acc[i][j][q]);
      }
    }
  }
}

bool gemm_nt_mfma_ok(const GemmArgs& g) {
  return g.M > 0 && g.N % kBN == 0 && g.K % kBK == 0 && g.K1 % kBK == 0 &&
         g.a1_k == 1 && g.a2_k == 1 && g.b_k == 1 && g.a1_m % 8 == 0 &&
         g.a2_m % 8 == 0 && g.b_n % 8 == 0;
}

hipError_t gemm_nt_mfma_launch(const GemmArgs& g, int c_type, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  dim3 grid(g.N / kBN, ceil_div(g.M, kBM));
  if (c_type == kBF16)
    gemm_nt_mfma_kernel<uint16_t><<<grid, 256, 0, s>>>(g);
  else
    gemm_nt_mfma_kernel<float><<<grid, 256, 0, s>>>(g);
  return hipGetLastError();
}

// ---------------------------------------------------------------- LayerNorm ---
template <typename T>
__global__ __launch_bounds__(256) void layernorm_rows_kernel(LnArgs a) {
  if (a.header[0] != 0) return;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.B) return;
  const float* u = a.U + static_cast<int64_t>(row) * a.d;
  float s = 0.f;
  for (int e = lane; e < a.d; e += 64) s += u[e];
  const float mean = wave_sum(s) / a.d;
  float q = 0.f;
  for (int e = lane; e < a.d; e += 64) {
    const float c = u[e] - mean;
    q += c * c;
  }
  const float var = wave_sum(q) / a.d;
  const float rstd = 1.0f / sqrtf(var + a.eps);
  const T* gamma = static_cast<const T*>(a.gamma);
  const T* beta = static_cast<const T*>(a.beta);
  T* h = static_cast<T*>(a.h);
  const int64_t base = static_cast<int64_t>(row) * a.d;
  for (int e = lane; e < a.d; e += 64) {
    const float uh = (u[e] - mean) * rstd;
    const float hv = ld<T>(gamma, e) * uh + ld<T>(beta, e);
    st<T>(h, base + e, hv);
    if (a.h_save) {
      a.h_save[base + e] = hv;
      a.uhat_save[base + e] = uh;
    }
  }
  if (a.rstd_save && lane == 0) a.rstd_save[row] = rstd;
}

hipError_t ln_launch(const LnArgs& a, int dtype, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  const int grid = ceil_div(a.B, 4);
  if (dtype == kBF16)
    layernorm_rows_kernel<uint16_t><<<grid, 256, 0, s>>>(a);
  else
    layernorm_rows_kernel<float><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace l3
