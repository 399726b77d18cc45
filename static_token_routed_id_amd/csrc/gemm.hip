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

// ------------------------------------------------- bf16 MFMA, 256 x 256 ---
// One workgroup (4 waves, one per SIMD) owns a 256 x 256 tile of C; wave
// (wm, wn) owns rows wm*128.. and columns wn*128.. as 4 x 4 blocks of
// 32x32x16 MFMA results (256 float accumulators per lane, in AGPRs). The K
// loop walks 64-wide slices: both operand slices (256 rows x 128 bytes)
// sit in LDS, double buffered (2 x 2 x 36 KB, rows padded to 72 elements so
// the 8 lanes served per LDS cycle hit distinct banks), and the slice two
// steps ahead is loaded from global memory into registers while the current
// one is multiplied, so one barrier per slice suffices. The prefetch is
// unconditional (clamped to the last slice) so the staging registers are
// never demoted to scratch memory.
//
// Tile order is XCD-aware: workgroup b runs on XCD b % 8, so tiles are
// renumbered to give each XCD a contiguous range of the logical order, which
// walks groups of 4 row-tiles x all column-tiles; the workgroups resident
// on one XCD at a time share A and B panels in that XCD's L2.
constexpr int kTM = 256, kTN = 256, kTK = 64, kTL = kTK + 8;
constexpr int kXcd = 8, kGroupM = 4;

template <typename TC, bool STATS>
__global__ __launch_bounds__(256, 1) void gemm_nt_256_kernel(GemmArgs g) {
  __shared__ uint16_t lds[2][2][kTM * kTL];
  if (g.header && g.header[0] != 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int mt = ceil_div(g.M, kTM), nt = g.N / kTN;
  const int T = mt * nt;
  int tile = blockIdx.x;
  if (T % kXcd == 0 && mt % kGroupM == 0)
    tile = (blockIdx.x % kXcd) * (T / kXcd) + blockIdx.x / kXcd;
  int m_tile, n_tile;
  if (mt % kGroupM == 0) {
    const int grp = tile / (kGroupM * nt), in = tile % (kGroupM * nt);
    m_tile = grp * kGroupM + in % kGroupM;
    n_tile = in / kGroupM;
  } else {
    m_tile = tile / nt;
    n_tile = tile % nt;
  }
  const int m0 = m_tile * kTM, n0 = n_tile * kTN;
  const uint16_t* A1 = static_cast<const uint16_t*>(g.A1);
  const uint16_t* A2 = static_cast<const uint16_t*>(g.A2);
  const uint16_t* Bm = static_cast<const uint16_t*>(g.Bm);

  // global -> register mapping: 8 lanes per 128-byte row slice, 32 rows per
  // pass, 8 passes per operand
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  int64_t aoff1[8], aoff2[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int64_t row = min(m0 + lr + 32 * q, g.M - 1);
    aoff1[q] = row * g.a1_m + lc;
    aoff2[q] = row * g.a2_m + lc;
  }
  const uint16_t* bbase = Bm + static_cast<int64_t>(n0 + lr) * g.b_n + lc;
  const int64_t bstep = 32 * g.b_n;
  u32x4 ra[8], rb[8];
#define L3_LOAD_SLICE(k0)                                                     \
  {                                                                           \
    const int kk0 = (k0);                                                     \
    const bool first = kk0 < g.K1;                                            \
    const uint16_t* ab = first ? A1 + kk0 : A2 + (kk0 - g.K1);                \
    _Pragma("unroll") for (int q = 0; q < 8; ++q) {                           \
      ra[q] = *reinterpret_cast<const u32x4*>(ab + (first ? aoff1[q]          \
                                                          : aoff2[q]));       \
      rb[q] = *reinterpret_cast<const u32x4*>(bbase + q * bstep + kk0);       \
    }                                                                         \
  }
#define L3_STORE_SLICE(buf)                                                   \
  {                                                                           \
    _Pragma("unroll") for (int q = 0; q < 8; ++q) {                           \
      *reinterpret_cast<u32x4*>(&lds[buf][0][(lr + 32 * q) * kTL + lc]) =     \
          ra[q];                                                              \
      *reinterpret_cast<u32x4*>(&lds[buf][1][(lr + 32 * q) * kTL + lc]) =     \
          rb[q];                                                              \
    }                                                                         \
  }

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};

  const int nk = g.K / kTK;
  const int r = lane & 31, kh = (lane >> 5) * 8;
  L3_LOAD_SLICE(0)
  L3_STORE_SLICE(0)
  L3_LOAD_SLICE(min(1, nk - 1) * kTK)
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const uint16_t* As = lds[it & 1][0] + (wm * 128 + r) * kTL + kh;
    const uint16_t* Bs = lds[it & 1][1] + (wn * 128 + r) * kTL + kh;
#pragma unroll
    for (int kk = 0; kk < kTK; kk += 16) {
      u32x4 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(As + i * 32 * kTL + kk);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const u32x4*>(Bs + j * 32 * kTL + kk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = mfma32_bf16(af[i], bf[j], acc[i][j]);
    }
    // the slice after next lands in the buffer just read; its global loads
    // overlap the next slice's multiplies (clamped: the tail reloads the
    // last slice into a buffer nobody reads again)
    L3_STORE_SLICE((it + 1) & 1)
    L3_LOAD_SLICE(min(it + 2, nk - 1) * kTK)
    __syncthreads();
  }
#undef L3_LOAD_SLICE
#undef L3_STORE_SLICE

  TC* C = static_cast<TC*>(g.C);
  const int h4 = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int gm = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + h4 + (e & 3);
      if (STATS) {
        // 128 columns of row gm live in this wave: 4 per lane across the 32
        // lanes of this half; mean and squared deviations of the float32
        // values (two passes over registers)
        float sm = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) sm += acc[i][j][e];
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) sm += __shfl_xor(sm, o);
        const float mean = sm * (1.0f / 128.0f);
        float m2 = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float c = acc[i][j][e] - mean;
          m2 += c * c;
        }
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) m2 += __shfl_xor(m2, o);
        if (r == 0 && gm < g.M) {
          const int chunk = (n0 + wn * 128) >> 7;
          *reinterpret_cast<float2*>(
              g.row_stats +
              (static_cast<int64_t>(gm) * (g.N >> 7) + chunk) * 2) =
              make_float2(mean, m2);
        }
      }
      if (gm >= g.M) continue;
      TC* crow = C + static_cast<int64_t>(gm) * g.c_m + n0 + wn * 128 + r;
#pragma unroll
      for (int j = 0; j < 4; ++j) st<TC>(crow, j * 32, acc[i][j][e]);
    }
  }
}

bool gemm_nt_256_ok(const GemmArgs& g) {
  return g.M >= 1024 && g.N % kTN == 0 && g.K % kTK == 0 &&
         g.K1 % kTK == 0 && g.a1_k == 1 && g.a2_k == 1 && g.b_k == 1 &&
         g.a1_m % 8 == 0 && g.a2_m % 8 == 0 && g.b_n % 8 == 0;
}

// ------------------------------------------------ LayerNorm from partials ---
// One wave per row: combine the row's per-128-column (mean, M2) partials with
// Chan's formula (equal chunk sizes), then h = gamma * (u - mean) * rstd +
// beta on 8 bf16 elements per lane and step.
__global__ __launch_bounds__(256) void ln_apply_kernel(LnApplyArgs a) {
  if (a.header[0] != 0) return;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.B) return;
  const int nch = a.d >> 7;
  const float* st = a.stats + static_cast<int64_t>(row) * nch * 2;
  float cm = 0.f, cq = 0.f;
  if (lane < nch) {
    const float2 v = *reinterpret_cast<const float2*>(st + 2 * lane);
    cm = v.x;
    cq = v.y;
  }
  const float mean = wave_sum(cm) / nch;
  const float dev = lane < nch ? (cm - mean) : 0.f;
  const float m2 = wave_sum(cq + 128.0f * dev * dev);
  const float rstd = 1.0f / sqrtf(m2 / a.d + a.eps);
  const int64_t base = static_cast<int64_t>(row) * a.d;
  for (int e0 = lane * 8; e0 < a.d; e0 += 512) {
    const uint4 u = *reinterpret_cast<const uint4*>(a.U + base + e0);
    const uint4 gv = *reinterpret_cast<const uint4*>(a.gamma + e0);
    const uint4 bv = *reinterpret_cast<const uint4*>(a.beta + e0);
    const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
    const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w};
    uint32_t ow[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float u0 = __uint_as_float(uw[q] << 16);
      const float u1 = __uint_as_float(uw[q] & 0xffff0000u);
      const float g0 = __uint_as_float(gw[q] << 16);
      const float g1 = __uint_as_float(gw[q] & 0xffff0000u);
      const float b0 = __uint_as_float(bw[q] << 16);
      const float b1 = __uint_as_float(bw[q] & 0xffff0000u);
      const float h0 = g0 * ((u0 - mean) * rstd) + b0;
      const float h1 = g1 * ((u1 - mean) * rstd) + b1;
      ow[q] = static_cast<uint32_t>(f2bf(h0)) |
              (static_cast<uint32_t>(f2bf(h1)) << 16);
    }
    *reinterpret_cast<uint4*>(a.h + base + e0) =
        make_uint4(ow[0], ow[1], ow[2], ow[3]);
  }
}

hipError_t ln_apply_launch(const LnApplyArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  ln_apply_kernel<<<ceil_div(a.B, 4), 256, 0, s>>>(a);
  return hipGetLastError();
}

bool gemm_nt_mfma_ok(const GemmArgs& g) {
  return g.M > 0 && g.N % kBN == 0 && g.K % kBK == 0 && g.K1 % kBK == 0 &&
         g.a1_k == 1 && g.a2_k == 1 && g.b_k == 1 && g.a1_m % 8 == 0 &&
         g.a2_m % 8 == 0 && g.b_n % 8 == 0;
}

hipError_t gemm_nt_mfma_launch(const GemmArgs& g, int c_type, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  if (gemm_nt_256_ok(g)) {
    const int grid = ceil_div(g.M, kTM) * (g.N / kTN);
    if (g.row_stats) {
      if (c_type != kBF16) return hipErrorInvalidValue;
      gemm_nt_256_kernel<uint16_t, true><<<grid, 256, 0, s>>>(g);
    } else if (c_type == kBF16) {
      gemm_nt_256_kernel<uint16_t, false><<<grid, 256, 0, s>>>(g);
    } else {
      gemm_nt_256_kernel<float, false><<<grid, 256, 0, s>>>(g);
    }
    return hipGetLastError();
  }
  if (g.row_stats) return hipErrorInvalidValue;
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
