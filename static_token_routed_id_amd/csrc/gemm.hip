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

#include <algorithm>

#include "l3_device.h"
#include "l3_internal.h"

namespace l3 {

// ---------------------------------------------------------------- generic ---
// Any strides, any mix of bf16 / float32 operands, float32 accumulation on
// 16x16x4 float32 MFMA. 64 x 64 tile per workgroup (four waves, 32 x 32
// each as 2 x 2 MFMA blocks), K in steps of 16 through double-buffered LDS;
// the next step's operands are loaded into registers while the current one
// is multiplied. Each operand is read along whichever of its dimensions is
// contiguous (16 consecutive k of a row, or 64 consecutive rows of a k).
// With nsplit > 1, workgroup z of the grid's third dimension takes the z-th
// share of K and writes its float32 partial product to part; gemm_reduce
// then adds the shares in order (the result does not depend on timing).
template <typename TA, typename TB, typename TC>
__global__ __launch_bounds__(256) void gemm_generic_kernel(GemmArgs g) {
  __shared__ float As[2][16][64 + 4];
  __shared__ float Bs[2][16][64 + 4];
  if (g.header && g.header[0] != 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int r = lane & 15, gq = lane >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const TA* A1 = static_cast<const TA*>(g.A1);
  const TA* A2 = static_cast<const TA*>(g.A2);
  const TB* Bm = static_cast<const TB*>(g.Bm);
  // this workgroup's share of K: [kbeg, kend), whole 16-steps
  const int kshare = ceil_div(ceil_div(g.K, g.nsplit), 16) * 16;
  const int kbeg = static_cast<int>(blockIdx.z) * kshare;
  const int kend = min(g.K, kbeg + kshare);
  // element q of this thread's share of a 16 x 64 operand slice
  const bool a_kfast = g.a1_k == 1 && g.a2_k == 1;
  const bool b_kfast = g.b_k == 1;
  auto a_pos = [&](int q, int& kk, int& mm) {
    const int e = tid + q * 256;
    if (a_kfast) {
      kk = e & 15;
      mm = e >> 4;
    } else {
      kk = e >> 6;
      mm = e & 63;
    }
  };
  auto b_pos = [&](int q, int& kk, int& nn) {
    const int e = tid + q * 256;
    if (b_kfast) {
      kk = e & 15;
      nn = e >> 4;
    } else {
      kk = e >> 6;
      nn = e & 63;
    }
  };
  float ra[4], rb[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int kk, mm;
      a_pos(q, kk, mm);
      const int gm = m0 + mm, gk = k0 + kk;
      float v = 0.f;
      if (gm < g.M && gk < kend) {
        v = gk < g.K1
                ? ld<TA>(A1, static_cast<int64_t>(gm) * g.a1_m +
                                 static_cast<int64_t>(gk) * g.a1_k)
                : ld<TA>(A2, static_cast<int64_t>(gm) * g.a2_m +
                                 static_cast<int64_t>(gk - g.K1) * g.a2_k);
      }
      ra[q] = v;
      int kb, nn;
      b_pos(q, kb, nn);
      const int gn = n0 + nn, gkb = k0 + kb;
      float bv = 0.f;
      if (gn < g.N && gkb < kend)
        bv = ld<TB>(Bm, static_cast<int64_t>(gkb) * g.b_k +
                            static_cast<int64_t>(gn) * g.b_n);
      rb[q] = bv;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int kk, mm;
      a_pos(q, kk, mm);
      As[buf][kk][mm] = ra[q];
      int kb, nn;
      b_pos(q, kb, nn);
      Bs[buf][kb][nn] = rb[q];
    }
  };
  floatx4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  load(kbeg);
  store(0);
  __syncthreads();
  const int nk = kend > kbeg ? ceil_div(kend - kbeg, 16) : 0;
  for (int it = 0; it < nk; ++it) {
    const int buf = it & 1;
    if (it + 1 < nk) load(kbeg + (it + 1) * 16);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k = ks * 4 + gq;
      float av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) av[i] = As[buf][k][wm * 32 + i * 16 + r];
#pragma unroll
      for (int j = 0; j < 2; ++j) bv[j] = Bs[buf][k][wn * 32 + j * 16 + r];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_f32(av[i], bv[j], acc[i][j]);
    }
    if (it + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }
  // D[4 gq + e][r] of block (i, j)
  TC* C = static_cast<TC*>(g.C);
  float* P = g.nsplit > 1
                 ? g.part + static_cast<int64_t>(blockIdx.z) * g.M * g.N
                 : nullptr;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int gm = m0 + wm * 32 + i * 16 + 4 * gq + e;
      if (gm >= g.M) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int gn = n0 + wn * 32 + j * 16 + r;
        if (gn < g.N) {
          if (P)
            P[static_cast<int64_t>(gm) * g.N + gn] = acc[i][j][e];
          else
            st<TC>(C, static_cast<int64_t>(gm) * g.c_m + gn, acc[i][j][e]);
        }
      }
    }
}

// Output v of the split-K sum: to C as TC, or, with lo (C bf16), as the
// bf16 pair hi = bf16(v) in C, lo = bf16(v - hi) in lo.
template <typename TC>
__device__ __forceinline__ void reduce_out(TC* c, uint16_t* lo, int64_t i,
                                           float v) {
  if constexpr (sizeof(TC) == 2) {
    if (lo) {
      const uint16_t h = f2bf(v);
      c[i] = h;
      lo[i] = f2bf(v - __uint_as_float(static_cast<uint32_t>(h) << 16));
      return;
    }
  }
  st<TC>(c, i, v);
}

// C = the nsplit partial products added in order (block blk of the
// reduction); with lo, as the bf16 hi | lo pair (reduce_out).
template <typename TC>
__device__ __forceinline__ void gemm_reduce_job(const GemmArgs& g, int blk,
                                                uint16_t* lo) {
  if (g.header && g.header[0] != 0) return;
  const int64_t mn = static_cast<int64_t>(g.M) * g.N;
  // four consecutive outputs a thread (16-byte loads) when N allows; the
  // shares are added in order z = 0, 1, ... whatever the loads' order
  if (g.N % 4 == 0) {
    const int64_t i = (static_cast<int64_t>(blk) * 256 + threadIdx.x) * 4;
    if (i >= mn) return;
    float4 v = {0.f, 0.f, 0.f, 0.f};
    const float* p = g.part + i;
    int z = 0;
    for (; z + 4 <= g.nsplit; z += 4) {
      float4 q[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        q[u] = *reinterpret_cast<const float4*>(p + (z + u) * mn);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v.x += q[u].x;
        v.y += q[u].y;
        v.z += q[u].z;
        v.w += q[u].w;
      }
    }
    for (; z < g.nsplit; ++z) {
      const float4 q = *reinterpret_cast<const float4*>(p + z * mn);
      v.x += q.x;
      v.y += q.y;
      v.z += q.z;
      v.w += q.w;
    }
    const int64_t m = i / g.N, n = i - m * g.N;
    TC* c = static_cast<TC*>(g.C);
    reduce_out<TC>(c, lo, m * g.c_m + n, v.x);
    reduce_out<TC>(c, lo, m * g.c_m + n + 1, v.y);
    reduce_out<TC>(c, lo, m * g.c_m + n + 2, v.z);
    reduce_out<TC>(c, lo, m * g.c_m + n + 3, v.w);
    return;
  }
  const int64_t i = static_cast<int64_t>(blk) * 256 + threadIdx.x;
  if (i >= mn) return;
  float v = 0.f;
  for (int z = 0; z < g.nsplit; ++z) v += g.part[z * mn + i];
  const int64_t m = i / g.N, n = i - m * g.N;
  reduce_out<TC>(static_cast<TC*>(g.C), lo, m * g.c_m + n, v);
}

template <typename TC>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmArgs g) {
  gemm_reduce_job<TC>(g, blockIdx.x, nullptr);
}

// The sums of two split-K products in one launch, both with bf16 C:
// blocks [0, n0) g0's, the rest g1's (with lo1: g1's as hi | lo).
__global__ __launch_bounds__(256) void gemm_reduce_pair_kernel(GemmArgs g0,
                                                               GemmArgs g1,
                                                               int n0,
                                                               uint16_t* lo1) {
  if (static_cast<int>(blockIdx.x) < n0)
    gemm_reduce_job<uint16_t>(g0, blockIdx.x, nullptr);
  else
    gemm_reduce_job<uint16_t>(g1, blockIdx.x - n0, lo1);
}

// grid of gemm_reduce_kernel for M x N outputs
static int reduce_grid(const GemmArgs& g) {
  const int64_t mn = static_cast<int64_t>(g.M) * g.N;
  const int64_t per = g.N % 4 == 0 ? 1024 : 256;
  return static_cast<int>((mn + per - 1) / per);
}

template <typename TA, typename TB>
static void gemm_generic_c(const GemmArgs& g, int c_type, dim3 grid,
                           hipStream_t s) {
  if (c_type == kBF16)
    gemm_generic_kernel<TA, TB, uint16_t><<<grid, 256, 0, s>>>(g);
  else
    gemm_generic_kernel<TA, TB, float><<<grid, 256, 0, s>>>(g);
}

hipError_t gemm_launch(const GemmArgs& g0, int a_type, int b_type, int c_type,
                       hipStream_t s, float* part, int64_t part_floats) {
  if (g0.M <= 0 || g0.N <= 0) return hipSuccess;
  GemmArgs g = g0;
  g.part = nullptr;
  g.nsplit = 1;
  // few output tiles and a long K (the weight gradients, K = tokens):
  // split K so that the GPU has enough workgroups
  const int64_t tiles =
      static_cast<int64_t>(ceil_div(g.N, 64)) * ceil_div(g.M, 64);
  const int64_t mn = static_cast<int64_t>(g.M) * g.N;
  if (part && tiles < 1024 && g.K >= 256) {
    int64_t ns = (1024 + tiles - 1) / tiles;
    ns = std::min<int64_t>(ns, g.K / 64);
    ns = std::min<int64_t>(ns, part_floats / mn);
    ns = std::min<int64_t>(ns, 64);
    if (ns >= 2) {
      g.part = part;
      g.nsplit = static_cast<int>(ns);
    }
  }
  dim3 grid(ceil_div(g.N, 64), ceil_div(g.M, 64), g.nsplit);
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
  if (g.nsplit > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int rgrid = reduce_grid(g);
    if (c_type == kBF16)
      gemm_reduce_kernel<uint16_t><<<rgrid, 256, 0, s>>>(g);
    else
      gemm_reduce_kernel<float><<<rgrid, 256, 0, s>>>(g);
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
// loop walks 64-wide slices, each split into four 16-wide steps:
//   * both operand slices (256 rows x 128 bytes) sit in LDS, double
//     buffered, rows padded to 72 elements so that a 16-byte read of 16 rows
//     touches 64 distinct banks;
//   * the fragments of step s+1 are read from LDS while the 16 MFMAs of step
//     s run (two fragment register sets); the first step of the next slice
//     is read after the workgroup barrier, during the last step's MFMAs;
//   * the slice after next is fetched from global memory into registers by
//     buffer loads (scalar base + 32-bit lane offset; rows past the matrix
//     end read as zero) and its previous contents written to the other LDS
//     buffer, spread over the first three steps: one load or LDS write
//     between consecutive MFMAs, never a burst that would stall the wave's
//     in-order issue behind a full memory queue.
// Scheduling barriers pin this interleaving; the compiler only inserts the
// waits each operand needs.
//
// Tile order is XCD-aware: workgroup b runs on XCD b % 8, so tiles are
// renumbered to give each XCD a contiguous range of the logical order, which
// walks groups of 4 row-tiles x all column-tiles; the workgroups resident
// on one XCD at a time share A and B panels in that XCD's L2.
//
// Options (GemmArgs): both operands switch source at k = K1 (A1 / A2, and
// B1 / Bm when B1 is set; b2_rel indexes Bm's columns from K1); K split over
// nsplit workgroups per tile into float32 partials (gemm_nt_256_splitk_
// launch); the LayerNorm fold, producer side (ln_stats_out: per-row sum and
// sum of squares of the tile after the stores) and consumer side (FOLD:
// per-row and per-column terms staged in LDS, one accumulator rescale
// between the k < K1 and k >= K1 loops, with explicit AGPR moves: a
// conditional rescale of the accumulators inside one loop made the register
// allocator spill, and a kernel with any spill runs several percent slower).
constexpr int kTM = 256, kTN = 256, kTK = 64, kTL = kTK + 8;
constexpr int kXcd = 8, kGroupM = 4;

struct Frag256 {
  u32x4 a[4], b[4];
};

// Operand source of one K slice: buffer resource, lane offset, row-group
// stride and slice column (all wave-uniform except the lane offset).
struct SliceSrc {
  __amdgpu_buffer_rsrc_t ra, rb;
  int va, vb, qa, qb, ka, kb;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(
    const uint16_t* base, int64_t bytes) {
  // 0x00020000: raw (untyped) 32-bit data format, the usual gfx9 setting
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(base), 0,
      static_cast<int>(bytes > 0x7fffffff ? 0x7fffffff : bytes), 0x00020000);
}

// One 16-wide step: 16 MFMAs on FC; after MFMA m, optionally the read of
// fragment m of the next step (m < 8) and staging operation m - S0 of rows
// Q0.. (per row group q: LDS write of A, of B, then reload of A, of B).
template <bool READ, int Q0, int NQ, int S0>
__device__ __forceinline__ void step256(floatx16 (&acc)[4][4],
                                        const Frag256& FC, Frag256& FN,
                                        const uint16_t* rd_a,
                                        const uint16_t* rd_b, int rd_k,
                                        u32x4 (&ra)[8], u32x4 (&rb)[8],
                                        uint16_t* wr_a, uint16_t* wr_b,
                                        const SliceSrc& src) {
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    acc[m >> 2][m & 3] = mfma32_bf16(FC.a[m >> 2], FC.b[m & 3],
                                     acc[m >> 2][m & 3]);
    if (READ && m < 8) {
      const int f = m >> 1;
      if (m & 1)
        FN.b[f] = *reinterpret_cast<const u32x4*>(rd_b + f * 32 * kTL + rd_k);
      else
        FN.a[f] = *reinterpret_cast<const u32x4*>(rd_a + f * 32 * kTL + rd_k);
    }
    if (m >= S0 && m - S0 < 4 * NQ) {
      const int q = Q0 + (m - S0) / 4, op = (m - S0) & 3;
      if (op == 0)
        *reinterpret_cast<u32x4*>(wr_a + q * 32 * kTL) = ra[q];
      else if (op == 1)
        *reinterpret_cast<u32x4*>(wr_b + q * 32 * kTL) = rb[q];
      else if (op == 2)
        ra[q] = __builtin_amdgcn_raw_buffer_load_b128(src.ra, src.va,
                                                      q * src.qa + src.ka, 0);
      else
        rb[q] = __builtin_amdgcn_raw_buffer_load_b128(src.rb, src.vb,
                                                      q * src.qb + src.kb, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One job (output tile and K share) of the 256 x 256 kernel; the kernel
// runs job blockIdx.x, the paired kernel below two products' jobs.
template <typename TC, bool FOLD, bool QUAD>
__device__ __forceinline__ void gemm256_job(const GemmArgs& g, int job) {
  __shared__ __align__(16) uint16_t lds[2][2][kTM * kTL];
  // LayerNorm fold (consumer): per tile row (rstd, -mean * rstd), per tile
  // column (c1, c2)
  __shared__ __align__(16) float2 s_rs[kTM];
  __shared__ __align__(16) float2 s_c[kTN];
  if (g.header && g.header[0] != 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int mt = ceil_div(g.M, kTM), nt = g.N / kTN;
  const int T = mt * nt;
  // split K (nsplit > 1, float32 partials): job b takes share b / T of K
  // for tile b % T
  const int kz = job / T, bt = job - kz * T;
  int tile = bt;
  if (T % kXcd == 0 && mt % kGroupM == 0)
    tile = (bt % kXcd) * (T / kXcd) + bt / kXcd;
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
  const int rows = min(kTM, g.M - m0);

  // global -> register mapping: 8 lanes per 128-byte row slice, 32 rows per
  // group, 8 groups per operand; the resources cover only this tile's rows
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  const __amdgpu_buffer_rsrc_t rA1 = make_rsrc(
      static_cast<const uint16_t*>(g.A1) + static_cast<int64_t>(m0) * g.a1_m,
      static_cast<int64_t>(rows) * g.a1_m * 2);
  const __amdgpu_buffer_rsrc_t rA2 = make_rsrc(
      static_cast<const uint16_t*>(g.A2) + static_cast<int64_t>(m0) * g.a2_m,
      static_cast<int64_t>(rows) * g.a2_m * 2);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(
      static_cast<const uint16_t*>(g.Bm) + static_cast<int64_t>(n0) * g.b_n,
      static_cast<int64_t>(kTN) * g.b_n * 2);
  // B operand of the k < K1 part (B1 if given, else Bm)
  const bool has_b1 = g.B1 != nullptr;
  const int64_t b1_n = has_b1 ? g.b1_n : g.b_n;
  const __amdgpu_buffer_rsrc_t rB1 =
      has_b1 ? make_rsrc(static_cast<const uint16_t*>(g.B1) +
                             static_cast<int64_t>(n0) * b1_n,
                         static_cast<int64_t>(kTN) * b1_n * 2)
             : rB;
  const int vA1 = static_cast<int>((lr * g.a1_m + lc) * 2);
  const int vA2 = static_cast<int>((lr * g.a2_m + lc) * 2);
  const int vB = static_cast<int>((lr * g.b_n + lc) * 2);
  const int vB1 = static_cast<int>((lr * b1_n + lc) * 2);
  const int qA1 = static_cast<int>(32 * g.a1_m * 2);
  const int qA2 = static_cast<int>(32 * g.a2_m * 2);
  const int qB = static_cast<int>(32 * g.b_n * 2);
  const int qB1 = static_cast<int>(32 * b1_n * 2);
  auto slice_src = [&](int k0) {
    SliceSrc s;
    const bool first = k0 < g.K1;
    s.ra = first ? rA1 : rA2;
    s.va = first ? vA1 : vA2;
    s.qa = first ? qA1 : qA2;
    s.ka = (first ? k0 : k0 - g.K1) * 2;
    s.rb = first ? rB1 : rB;
    s.vb = first ? vB1 : vB;
    s.qb = first ? qB1 : qB;
    s.kb = (first || !g.b2_rel ? k0 : k0 - g.K1) * 2;
    return s;
  };

  // LayerNorm fold (consumer): the row's (rstd, -mean * rstd) and the
  // column's (c1, c2), loaded before the first operand slice
  constexpr bool fold = FOLD;
  float2 lnr = make_float2(0.f, 0.f), lnc = make_float2(0.f, 0.f);
  if constexpr (FOLD) {
    if (m0 + tid < g.M)
      lnr = reinterpret_cast<const float2*>(g.ln_rows)[m0 + tid];
    lnc = reinterpret_cast<const float2*>(g.ln_c12)[n0 + tid];
  }

  u32x4 ra[8], rb[8];
  auto load_all = [&](const SliceSrc& s) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      ra[q] = __builtin_amdgcn_raw_buffer_load_b128(s.ra, s.va, q * s.qa + s.ka,
                                                    0);
      rb[q] = __builtin_amdgcn_raw_buffer_load_b128(s.rb, s.vb, q * s.qb + s.kb,
                                                    0);
    }
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};

  const int kshare = g.K / g.nsplit;
  const int kbeg = kz * kshare;
  const int nk = kshare / kTK;
  const int r = lane & 31, kh = (lane >> 5) * 8;
  const int aoff = (wm * 128 + r) * kTL + kh, boff = (wn * 128 + r) * kTL + kh;
  const int woff = lr * kTL + lc;
  load_all(slice_src(kbeg));
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    *reinterpret_cast<u32x4*>(&lds[0][0][woff + q * 32 * kTL]) = ra[q];
    *reinterpret_cast<u32x4*>(&lds[0][1][woff + q * 32 * kTL]) = rb[q];
  }
  if constexpr (FOLD) {
    s_rs[tid] = lnr;
    s_c[tid] = lnc;
  }
  load_all(slice_src(kbeg + min(1, nk - 1) * kTK));
  __syncthreads();
  Frag256 F0, F1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    F0.a[i] = *reinterpret_cast<const u32x4*>(&lds[0][0][aoff + i * 32 * kTL]);
    F0.b[i] = *reinterpret_cast<const u32x4*>(&lds[0][1][boff + i * 32 * kTL]);
  }
  auto kslice = [&](int it) __attribute__((always_inline)) {
    const int buf = it & 1;
    // slice it+1 (in registers) goes to the other buffer, slice it+2 is
    // fetched (clamped: the tail refetches the last slice, never read)
    const SliceSrc src = slice_src(kbeg + min(it + 2, nk - 1) * kTK);
    const uint16_t* rda = &lds[buf][0][aoff];
    const uint16_t* rdb = &lds[buf][1][boff];
    uint16_t* wra = &lds[buf ^ 1][0][woff];
    uint16_t* wrb = &lds[buf ^ 1][1][woff];
    step256<true, 0, 3, 4>(acc, F0, F1, rda, rdb, 16, ra, rb, wra, wrb, src);
    step256<true, 3, 3, 4>(acc, F1, F0, rda, rdb, 32, ra, rb, wra, wrb, src);
    step256<true, 6, 2, 8>(acc, F0, F1, rda, rdb, 48, ra, rb, wra, wrb, src);
    __syncthreads();
    step256<true, 0, 0, 16>(acc, F1, F0, &lds[buf ^ 1][0][aoff],
                            &lds[buf ^ 1][1][boff], 0, ra, rb, wra, wrb, src);
  };
  // with the fold, the k < K1 part runs first, then the accumulators take
  // the LayerNorm terms, then the rest
  const int nk1 = FOLD ? g.K1 / kTK : nk;
  int it = 0;
  for (; it < nk1; ++it) kslice(it);
  if constexpr (FOLD) {
    // acc = rstd * acc - mean * rstd * c1 + c2, four rows of a 32 x 32
    // block at a time; each value is moved out of its AGPR and back by
    // explicit moves (left to the register allocator, the rescaled values
    // crowd the VGPRs and spill)
    float2 c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = s_c[wn * 128 + j * 32 + r];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int eg = 0; eg < 4; ++eg) {
        // rows wm*128 + i*32 + 8*eg + h .. +3 (h = 0 or 4 by lane half)
        const float4* rs4 = reinterpret_cast<const float4*>(
            &s_rs[wm * 128 + i * 32 + 8 * eg + (lane >> 5) * 4]);
        const float4 r01 = rs4[0], r23 = rs4[1];
        const float ra4[4] = {r01.x, r01.z, r23.x, r23.z};
        const float rb4[4] = {r01.y, r01.w, r23.y, r23.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int ee = 0; ee < 4; ++ee) {
            float v;
            asm volatile("v_accvgpr_read_b32 %0, %1"
                         : "=v"(v)
                         : "a"(acc[i][j][4 * eg + ee]));
            v = fmaf(ra4[ee], v, fmaf(rb4[ee], c[j].x, c[j].y));
            float o;
            asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(o) : "v"(v));
            acc[i][j][4 * eg + ee] = o;
          }
        }
      }
  }
  for (; it < nk; ++it) kslice(it);

  const int h4 = (lane >> 5) * 4;

  // split K: share kz's partial product, M x N float32 (the launcher takes
  // this path for float32 C only)
  TC* C = g.nsplit > 1 ? reinterpret_cast<TC*>(g.part) +
                             static_cast<int64_t>(kz) * g.M * g.N
                       : static_cast<TC*>(g.C);
  const int64_t c_m = g.nsplit > 1 ? g.N : g.c_m;
#pragma unroll
  for (int i = 0; i < (QUAD ? 0 : 4); ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int gm = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + h4 + (e & 3);
      if (gm >= g.M) continue;
      TC* crow = C + static_cast<int64_t>(gm) * c_m + n0 + wn * 128 + r;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // streaming (non-temporal) stores: C is read much later or by a
        // kernel that streams it once; kept out of the caches, it does not
        // evict operands, and the write-back does not delay what follows
        if constexpr (sizeof(TC) == 4)
          __builtin_nontemporal_store(acc[i][j][e],
                                      reinterpret_cast<float*>(crow) + j * 32);
        else
          __builtin_nontemporal_store(
              f2bf(acc[i][j][e]), reinterpret_cast<uint16_t*>(crow) + j * 32);
      }
    }
  }

  if (!FOLD && (QUAD || g.ln_stats_out)) {
    // LayerNorm fold (producer): sum and sum of squares of each tile row
    // over the tile's 256 columns, then (mean, M2 = sum of squares - sum *
    // mean) in float32 (one pass; M2 is exact to float32 rounding of the
    // sums while |mean| / std stays well below 2^12). Each lane first adds
    // up its four columns of a row; the 64 lane sums of a row (32 lanes x
    // 2 waves) meet in LDS as [slot][row] (row stride padded by 4 floats:
    // the float4 writes of 8 lanes fall in distinct banks) and one thread
    // a row adds them up.
    constexpr int kSP = kTM + 4;
    // quadratic form: Q's tile rows staged in LDS half a tile (128 rows) at
    // a time, [128][kQL] bf16 ahead of the sums (sq); else sums at sp, sq
    constexpr int kQL = kTN + 8;
    float* sp = reinterpret_cast<float*>(&lds[0][0][0]);
    float* sq = QUAD ? reinterpret_cast<float*>(
                           reinterpret_cast<uint16_t*>(sp) + 128 * kQL)
                     : sp + 64 * kSP;
    uint16_t* qs = reinterpret_cast<uint16_t*>(sp);
    static_assert(128 * kQL * 2 + 64 * kSP * 4 <= sizeof(lds),
                  "quadratic-form staging exceeds the operand LDS");
    const int wo = (wn * 32 + r) * kSP + wm * 128 + h4;
    // quadratic form: Q's tile rows, 128 at a time, as 8 rows a pass of
    // 16-byte chunks; a thread's sixteen loads are all in flight before its
    // first LDS write, and the second half's are issued before the first
    // half's products
    const int qc = (tid & 31) * 8;
    u32x4 qv[QUAD ? 16 : 1];
    auto load_q = [&](int half) {
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        const int gm = min(m0 + half * 128 + p * 8 + (tid >> 5), g.M - 1);
        qv[p] = *reinterpret_cast<const u32x4*>(
            g.ln_quad_a + static_cast<int64_t>(gm) * g.ln_quad_lda + n0 + qc);
      }
    };
    if constexpr (QUAD) load_q(0);
    __syncthreads();  // every wave is done with the operand buffers
#pragma unroll
    for (int half = 0; half < (QUAD ? 2 : 1); ++half) {
    if constexpr (QUAD) {
      if (half > 0) __syncthreads();  // the first half's products are done
#pragma unroll
      for (int p = 0; p < 16; ++p)
        *reinterpret_cast<u32x4*>(&qs[(p * 8 + (tid >> 5)) * kQL + qc]) =
            qv[p];
      if (half == 0) load_q(1);
      __syncthreads();
      if (wm != half) continue;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int eg = 0; eg < 4; ++eg) {
        float4 v, w;
        float* vp = reinterpret_cast<float*>(&v);
        float* wp = reinterpret_cast<float*>(&w);
        if constexpr (QUAD) {
          // the tile rows times Q's entries at the same positions (rows
          // past M took row M - 1; never written): the sixteen entries
          // this lane needs (four rows, four columns) are read first, then
          // the accumulators by explicit AGPR reads, as in the fold above
          // (left to the allocator, part of acc moved to VGPRs and this
          // epilogue ran with a handful of free registers, each LDS read
          // waited for before the next: the kernel took 104 us, now 79)
          float q[4][4];
#pragma unroll
          for (int ee = 0; ee < 4; ++ee) {
            const uint16_t* qrow =
                qs + (i * 32 + 8 * eg + h4 + ee) * kQL + wn * 128 + r;
#pragma unroll
            for (int j = 0; j < 4; ++j) q[ee][j] = bf2f(qrow[j * 32]);
          }
#pragma unroll
          for (int ee = 0; ee < 4; ++ee) {
            float b = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              float x;
              asm volatile("v_accvgpr_read_b32 %0, %1"
                           : "=v"(x)
                           : "a"(acc[i][j][4 * eg + ee]));
              b = fmaf(x, q[ee][j], b);
            }
            vp[ee] = 0.f;
            wp[ee] = b;
          }
        } else {
#pragma unroll
          for (int ee = 0; ee < 4; ++ee) {
            float a = 0.f, b = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float x = acc[i][j][4 * eg + ee];
              a += x;
              b = fmaf(x, x, b);
            }
            vp[ee] = a;
            wp[ee] = b;
          }
        }
        if constexpr (!QUAD)
          *reinterpret_cast<float4*>(sp + wo + i * 32 + 8 * eg) = v;
        *reinterpret_cast<float4*>(sq + wo + i * 32 + 8 * eg) = w;
      }
    }
    __syncthreads();
    float sum = 0.f, sum2 = 0.f;
#pragma unroll 16
    for (int sl = 0; sl < 64; ++sl) {
      if constexpr (!QUAD) sum += sp[sl * kSP + tid];
      sum2 += sq[sl * kSP + tid];
    }
    const float mean = sum * (1.0f / kTN);
    const float m2 = fmaxf(sum2 - sum * mean, 0.f);
    if (m0 + tid < g.M)
      reinterpret_cast<float2*>(g.ln_stats_out)[static_cast<int64_t>(m0 + tid) *
                                                    nt + n_tile] =
          QUAD ? make_float2(sum2, 0.f) : make_float2(mean, m2);
  }
}

template <typename TC, bool FOLD, bool QUAD = false>
__global__ __launch_bounds__(256, 1) void gemm_nt_256_kernel(GemmArgs g) {
  gemm256_job<TC, FOLD, QUAD>(g, blockIdx.x);
}

// Two split-K products (float32 partials) in one launch: workgroups
// [0, n0) take g0's jobs, the rest g1's (the job's LDS is the same
// function's, so the two share it).
__global__ __launch_bounds__(256, 1) void gemm_nt_256_pair_kernel(GemmArgs g0,
                                                                 GemmArgs g1,
                                                                 int n0) {
  if (static_cast<int>(blockIdx.x) < n0)
    gemm256_job<float, false, false>(g0, blockIdx.x);
  else
    gemm256_job<float, false, false>(g1, blockIdx.x - n0);
}

// ------------------------------- bf16 MFMA, 256 (or 128) x 256, eight waves ---
// The same slice pipeline and LDS layout as the four-wave kernel above,
// with eight waves (two a SIMD): wave (wm, wn), wm < 2, wn < 4, owns rows
// wm*32*MI.. and columns wn*64.. as MI x 2 blocks of 32x32x16 MFMA results
// (32 MI float accumulators a lane). MI = 4 is a 256 x 256 tile; MI = 2 a
// 128 x 256 tile, for products with too few 256 x 256 tiles to fill the
// GPU. With two waves on each SIMD one wave's MFMAs run while the other
// waits for its LDS fragments or the barrier; the LDS reads per slice grow
// by half (each A fragment is read by four waves instead of two), within
// gfx950's LDS rate. Each 16-wide step is 2 MI MFMAs; the next step's
// fragments are read during the first MI + 2 of them, and the next slice
// (512 threads: 16-byte chunks of 64-row groups, MI of A and four of B) is
// staged one LDS write or buffer load after each MFMA over the first steps
// (per A group: write A, write B, reload A, reload B; then the remaining B
// groups: write, reload). Plain float32 or bf16 C, optionally the LayerNorm
// fold (consumer side); no split K and no producer-side statistics (those
// stay on the four-wave kernel).
template <int MI>
struct FragW8 {
  u32x4 a[MI], b[2];
};

// The t-th staging operation of a slice: (row group q, kind): 0 write A,
// 1 write B, 2 reload A, 3 reload B.
template <int MI>
__device__ __forceinline__ constexpr int w8_nops() {
  return 4 * MI + 2 * (4 - MI);
}

template <int MI, bool READ, int T0>
__device__ __forceinline__ void step_w8(floatx16 (&acc)[MI][2],
                                        const FragW8<MI>& FC, FragW8<MI>& FN,
                                        const uint16_t* rd_a,
                                        const uint16_t* rd_b, int rd_k,
                                        u32x4 (&ra)[MI], u32x4 (&rb)[4],
                                        uint16_t* wr_a, uint16_t* wr_b,
                                        const SliceSrc& src) {
#pragma unroll
  for (int m = 0; m < 2 * MI; ++m) {
    acc[m >> 1][m & 1] = mfma32_bf16(FC.a[m >> 1], FC.b[m & 1],
                                     acc[m >> 1][m & 1]);
    if (READ && m < MI)
      FN.a[m] = *reinterpret_cast<const u32x4*>(rd_a + m * 32 * kTL + rd_k);
    else if (READ && m < MI + 2)
      FN.b[m - MI] =
          *reinterpret_cast<const u32x4*>(rd_b + (m - MI) * 32 * kTL + rd_k);
    const int t = T0 + m;
    if (t < w8_nops<MI>()) {
      int q, op;
      if (t < 4 * MI) {
        q = t / 4;
        op = t & 3;
      } else {
        q = MI + (t - 4 * MI) / 2;
        op = ((t - 4 * MI) & 1) ? 3 : 1;
      }
      if (op == 0)
        *reinterpret_cast<u32x4*>(wr_a + q * 64 * kTL) = ra[q];
      else if (op == 1)
        *reinterpret_cast<u32x4*>(wr_b + q * 64 * kTL) = rb[q];
      else if (op == 2)
        ra[q] = __builtin_amdgcn_raw_buffer_load_b128(src.ra, src.va,
                                                      q * src.qa + src.ka, 0);
      else
        rb[q] = __builtin_amdgcn_raw_buffer_load_b128(src.rb, src.vb,
                                                      q * src.qb + src.kb, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <typename TC, bool FOLD, int MI, bool STATS = false>
__global__ __launch_bounds__(512, 1) void gemm_nt_256w8_kernel(GemmArgs g) {
  constexpr int TM = 64 * MI;  // tile rows
  __shared__ __align__(16) uint16_t lds[2][2][kTM * kTL];
  __shared__ __align__(16) float2 s_rs[TM];
  __shared__ __align__(16) float2 s_c[kTN];
  if (g.header && g.header[0] != 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int mt = ceil_div(g.M, TM), nt = g.N / kTN;
  const int T = mt * nt;
  const int bt = blockIdx.x;
  int tile = bt;
  if (T % kXcd == 0 && mt % kGroupM == 0)
    tile = (bt % kXcd) * (T / kXcd) + bt / kXcd;
  int m_tile, n_tile;
  if (mt % kGroupM == 0) {
    const int grp = tile / (kGroupM * nt), in = tile % (kGroupM * nt);
    m_tile = grp * kGroupM + in % kGroupM;
    n_tile = in / kGroupM;
  } else {
    m_tile = tile / nt;
    n_tile = tile % nt;
  }
  const int m0 = m_tile * TM, n0 = n_tile * kTN;
  const int rows = min(TM, g.M - m0);

  // global -> register mapping: 8 lanes per 128-byte row slice, 64 rows per
  // group; MI groups of A, 4 of B
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  const __amdgpu_buffer_rsrc_t rA1 = make_rsrc(
      static_cast<const uint16_t*>(g.A1) + static_cast<int64_t>(m0) * g.a1_m,
      static_cast<int64_t>(rows) * g.a1_m * 2);
  const __amdgpu_buffer_rsrc_t rA2 = make_rsrc(
      static_cast<const uint16_t*>(g.A2) + static_cast<int64_t>(m0) * g.a2_m,
      static_cast<int64_t>(rows) * g.a2_m * 2);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(
      static_cast<const uint16_t*>(g.Bm) + static_cast<int64_t>(n0) * g.b_n,
      static_cast<int64_t>(kTN) * g.b_n * 2);
  const bool has_b1 = g.B1 != nullptr;
  const int64_t b1_n = has_b1 ? g.b1_n : g.b_n;
  const __amdgpu_buffer_rsrc_t rB1 =
      has_b1 ? make_rsrc(static_cast<const uint16_t*>(g.B1) +
                             static_cast<int64_t>(n0) * b1_n,
                         static_cast<int64_t>(kTN) * b1_n * 2)
             : rB;
  const int vA1 = static_cast<int>((lr * g.a1_m + lc) * 2);
  const int vA2 = static_cast<int>((lr * g.a2_m + lc) * 2);
  const int vB = static_cast<int>((lr * g.b_n + lc) * 2);
  const int vB1 = static_cast<int>((lr * b1_n + lc) * 2);
  const int qA1 = static_cast<int>(64 * g.a1_m * 2);
  const int qA2 = static_cast<int>(64 * g.a2_m * 2);
  const int qB = static_cast<int>(64 * g.b_n * 2);
  const int qB1 = static_cast<int>(64 * b1_n * 2);
  auto slice_src = [&](int k0) {
    SliceSrc s;
    const bool first = k0 < g.K1;
    s.ra = first ? rA1 : rA2;
    s.va = first ? vA1 : vA2;
    s.qa = first ? qA1 : qA2;
    s.ka = (first ? k0 : k0 - g.K1) * 2;
    s.rb = first ? rB1 : rB;
    s.vb = first ? vB1 : vB;
    s.qb = first ? qB1 : qB;
    s.kb = (first || !g.b2_rel ? k0 : k0 - g.K1) * 2;
    return s;
  };

  float2 lnr = make_float2(0.f, 0.f), lnc = make_float2(0.f, 0.f);
  if constexpr (FOLD) {
    if (tid < TM && m0 + tid < g.M)
      lnr = reinterpret_cast<const float2*>(g.ln_rows)[m0 + tid];
    if (tid < kTN) lnc = reinterpret_cast<const float2*>(g.ln_c12)[n0 + tid];
  }

  u32x4 ra[MI], rb[4];
  auto load_all = [&](const SliceSrc& s) {
#pragma unroll
    for (int q = 0; q < MI; ++q)
      ra[q] = __builtin_amdgcn_raw_buffer_load_b128(s.ra, s.va, q * s.qa + s.ka,
                                                    0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      rb[q] = __builtin_amdgcn_raw_buffer_load_b128(s.rb, s.vb, q * s.qb + s.kb,
                                                    0);
  };

  floatx16 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{};

  const int nk = g.K / kTK;
  const int r = lane & 31, kh = (lane >> 5) * 8;
  const int aoff = (wm * 32 * MI + r) * kTL + kh,
            boff = (wn * 64 + r) * kTL + kh;
  const int woff = lr * kTL + lc;
  load_all(slice_src(0));
#pragma unroll
  for (int q = 0; q < MI; ++q)
    *reinterpret_cast<u32x4*>(&lds[0][0][woff + q * 64 * kTL]) = ra[q];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<u32x4*>(&lds[0][1][woff + q * 64 * kTL]) = rb[q];
  if constexpr (FOLD) {
    if (tid < TM) s_rs[tid] = lnr;
    if (tid < kTN) s_c[tid] = lnc;
  }
  load_all(slice_src(min(1, nk - 1) * kTK));
  __syncthreads();
  FragW8<MI> F0, F1;
#pragma unroll
  for (int i = 0; i < MI; ++i)
    F0.a[i] = *reinterpret_cast<const u32x4*>(&lds[0][0][aoff + i * 32 * kTL]);
#pragma unroll
  for (int j = 0; j < 2; ++j)
    F0.b[j] = *reinterpret_cast<const u32x4*>(&lds[0][1][boff + j * 32 * kTL]);
  constexpr int kOps = 2 * MI;  // staging operations a step
  auto kslice = [&](int it) __attribute__((always_inline)) {
    const int buf = it & 1;
    // slice it+1 (in registers) goes to the other buffer, slice it+2 is
    // fetched (clamped: the tail refetches the last slice, never read)
    const SliceSrc src = slice_src(min(it + 2, nk - 1) * kTK);
    const uint16_t* rda = &lds[buf][0][aoff];
    const uint16_t* rdb = &lds[buf][1][boff];
    uint16_t* wra = &lds[buf ^ 1][0][woff];
    uint16_t* wrb = &lds[buf ^ 1][1][woff];
    step_w8<MI, true, 0>(acc, F0, F1, rda, rdb, 16, ra, rb, wra, wrb, src);
    step_w8<MI, true, kOps>(acc, F1, F0, rda, rdb, 32, ra, rb, wra, wrb,
                            src);
    step_w8<MI, true, 2 * kOps>(acc, F0, F1, rda, rdb, 48, ra, rb, wra, wrb,
                                src);
    __syncthreads();
    step_w8<MI, true, 64>(acc, F1, F0, &lds[buf ^ 1][0][aoff],
                          &lds[buf ^ 1][1][boff], 0, ra, rb, wra, wrb, src);
  };
  static_assert(w8_nops<MI>() <= 3 * 2 * MI,
                "a slice's staging fits in its first three steps");
  const int nk1 = FOLD ? g.K1 / kTK : nk;
  int it = 0;
  for (; it < nk1; ++it) kslice(it);
  if constexpr (FOLD) {
    // acc = rstd * acc - mean * rstd * c1 + c2 (explicit AGPR moves, as in
    // the four-wave kernel)
    float2 c[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) c[j] = s_c[wn * 64 + j * 32 + r];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int eg = 0; eg < 4; ++eg) {
        const float4* rs4 = reinterpret_cast<const float4*>(
            &s_rs[wm * 32 * MI + i * 32 + 8 * eg + (lane >> 5) * 4]);
        const float4 r01 = rs4[0], r23 = rs4[1];
        const float ra4[4] = {r01.x, r01.z, r23.x, r23.z};
        const float rb4[4] = {r01.y, r01.w, r23.y, r23.w};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int ee = 0; ee < 4; ++ee) {
            float v;
            asm volatile("v_accvgpr_read_b32 %0, %1"
                         : "=v"(v)
                         : "a"(acc[i][j][4 * eg + ee]));
            v = fmaf(ra4[ee], v, fmaf(rb4[ee], c[j].x, c[j].y));
            float o;
            asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(o) : "v"(v));
            acc[i][j][4 * eg + ee] = o;
          }
        }
      }
  }
  for (; it < nk; ++it) kslice(it);

  const int h4 = (lane >> 5) * 4;
  TC* C = static_cast<TC*>(g.C);
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int gm = m0 + wm * 32 * MI + i * 32 + 8 * (e >> 2) + h4 + (e & 3);
      if (gm >= g.M) continue;
      TC* crow = C + static_cast<int64_t>(gm) * g.c_m + n0 + wn * 64 + r;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (sizeof(TC) == 4)
          __builtin_nontemporal_store(acc[i][j][e],
                                      reinterpret_cast<float*>(crow) + j * 32);
        else
          __builtin_nontemporal_store(
              f2bf(acc[i][j][e]), reinterpret_cast<uint16_t*>(crow) + j * 32);
      }
    }
  }
  if constexpr (STATS) {
    // LayerNorm fold (producer): each tile row's sum and sum of squares over
    // the tile's 256 columns (the float32 accumulators) as (mean, M2 = sum
    // of squares - sum * mean; one pass, exact to float32 rounding while
    // |mean| / std stays well below 2^12). The 128 lane sums of a row (32
    // lanes x 4 column waves) meet in the operand LDS as [slot][row] (row
    // stride padded by 4 floats: each float4 write of 4 rows falls in its
    // own banks); one thread a row adds them up in slot order.
    constexpr int kSP = TM + 4;
    float* sp = reinterpret_cast<float*>(&lds[0][0][0]);
    float* sq = sp + 128 * kSP;
    static_assert(2 * 128 * kSP * 4 <= sizeof(lds),
                  "row-sum slots exceed the operand LDS");
    __syncthreads();  // every wave is done with the operand buffers
    const int wo = (wn * 32 + r) * kSP + wm * 32 * MI + h4;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int eg = 0; eg < 4; ++eg) {
        float4 v, w2;
        float* vp = reinterpret_cast<float*>(&v);
        float* wp = reinterpret_cast<float*>(&w2);
#pragma unroll
        for (int ee = 0; ee < 4; ++ee) {
          const float x0 = acc[i][0][4 * eg + ee], x1 = acc[i][1][4 * eg + ee];
          vp[ee] = x0 + x1;
          wp[ee] = fmaf(x0, x0, x1 * x1);
        }
        *reinterpret_cast<float4*>(sp + wo + i * 32 + 8 * eg) = v;
        *reinterpret_cast<float4*>(sq + wo + i * 32 + 8 * eg) = w2;
      }
    __syncthreads();
    if (tid < TM) {
      float sum = 0.f, sum2 = 0.f;
#pragma unroll 16
      for (int sl = 0; sl < 128; ++sl) {
        sum += sp[sl * kSP + tid];
        sum2 += sq[sl * kSP + tid];
      }
      const float mean = sum * (1.0f / kTN);
      const float m2 = fmaxf(sum2 - sum * mean, 0.f);
      if (m0 + tid < g.M)
        reinterpret_cast<float2*>(g.ln_stats_out)[static_cast<int64_t>(m0 +
                                                                   tid) *
                                                      nt + n_tile] =
            make_float2(mean, m2);
    }
  }
}

// Shape rules of the 256 x 256 kernel; gemm_nt_256_ok adds M >= 1024 (below
// that the launcher prefers other tilings, or the split-K form for few rows).
static bool gemm_nt_256_shape_ok(const GemmArgs& g) {
  // buffer offsets are 32-bit: one tile's rows must span < 2 GiB
  return g.M > 0 && g.N % kTN == 0 && g.K % kTK == 0 &&
         g.K1 % kTK == 0 && g.a1_k == 1 && g.a2_k == 1 && g.b_k == 1 &&
         g.a1_m % 8 == 0 && g.a2_m % 8 == 0 && g.b_n % 8 == 0 &&
         static_cast<int64_t>(kTM) * g.a1_m * 2 < (int64_t(1) << 30) &&
         static_cast<int64_t>(kTM) * g.a2_m * 2 < (int64_t(1) << 30) &&
         static_cast<int64_t>(kTN) * g.b_n * 2 < (int64_t(1) << 30);
}

bool gemm_nt_256_ok(const GemmArgs& g) {
  return g.M >= 1024 && gemm_nt_256_shape_ok(g);
}

// The 256 x 256 kernel with K split over up to max_split workgroups (few
// output tiles and a long K: the weight gradients, K = tokens), about 256
// workgroups in all, float32 C: each share writes
// its partial product to part, then gemm_reduce_kernel adds the shares in
// order. Returns hipErrorInvalidValue when the shape does not allow it
// (the caller then takes another path).
// K shares of a split-K launch: about 256 workgroups in all, at most
// max_split, whole 64-wide slices in every share (a share may straddle K1:
// the operands switch per slice), the partials within part_floats.
static int splitk_shares(const GemmArgs& g, int max_split,
                         int64_t part_floats) {
  const int64_t tiles =
      static_cast<int64_t>(ceil_div(g.M, kTM)) * (g.N / kTN);
  const int64_t mn = static_cast<int64_t>(g.M) * g.N;
  int ns = static_cast<int>(
      std::min<int64_t>((256 + tiles - 1) / tiles, max_split));
  while (ns > 1 && ((g.K % (ns * kTK)) != 0 || ns * mn > part_floats))
    --ns;
  return ns;
}

hipError_t gemm_nt_256_splitk_launch(const GemmArgs& g0, hipStream_t s,
                                     float* part, int64_t part_floats,
                                     int max_split, int c_type) {
  if (!gemm_nt_256_shape_ok(g0)) return hipErrorInvalidValue;
  if (!part) part_floats = 0;
  GemmArgs g = g0;
  const int64_t tiles =
      static_cast<int64_t>(ceil_div(g.M, kTM)) * (g.N / kTN);
  const int ns = splitk_shares(g, max_split, part_floats);
  g.nsplit = ns;
  g.part = ns > 1 ? part : nullptr;
  const int grid = static_cast<int>(tiles) * ns;
  // the shares' partials are float32 whatever C is; one share writes C
  if (ns > 1 || c_type != kBF16)
    gemm_nt_256_kernel<float, false><<<grid, 256, 0, s>>>(g);
  else
    gemm_nt_256_kernel<uint16_t, false><<<grid, 256, 0, s>>>(g);
  if (ns > 1) {
    const int rgrid = reduce_grid(g);
    if (c_type == kBF16)
      gemm_reduce_kernel<uint16_t><<<rgrid, 256, 0, s>>>(g);
    else
      gemm_reduce_kernel<float><<<rgrid, 256, 0, s>>>(g);
  }
  return hipGetLastError();
}

// Two independent products as gemm_nt_256_splitk_launch would run them (the
// same K shares, so the same sums), in one launch of both products' jobs
// and one of both sums: a's C as bf16, b's as the bf16 pair C (hi) and b_lo
// (lo) of its float32 sum. a's partials come first in part, then b's.
// Returns hipErrorInvalidValue (nothing launched) unless both shapes allow
// the 256 x 256 kernel and both split in two or more shares.
hipError_t gemm_nt_256_splitk_pair_launch(const GemmArgs& a0, int max_a,
                                          const GemmArgs& b0, int max_b,
                                          uint16_t* b_lo, float* part,
                                          int64_t part_floats, hipStream_t s) {
  if (!part || !b_lo || !gemm_nt_256_shape_ok(a0) ||
      !gemm_nt_256_shape_ok(b0))
    return hipErrorInvalidValue;
  GemmArgs a = a0, b = b0;
  const int64_t mn_a = static_cast<int64_t>(a.M) * a.N;
  a.nsplit = splitk_shares(a, max_a, part_floats);
  const int64_t left = part_floats - a.nsplit * mn_a;
  b.nsplit = splitk_shares(b, max_b, left);
  if (a.nsplit < 2 || b.nsplit < 2) return hipErrorInvalidValue;
  a.part = part;
  b.part = part + a.nsplit * mn_a;
  const int jobs_a = ceil_div(a.M, kTM) * (a.N / kTN) * a.nsplit;
  const int jobs_b = ceil_div(b.M, kTM) * (b.N / kTN) * b.nsplit;
  gemm_nt_256_pair_kernel<<<jobs_a + jobs_b, 256, 0, s>>>(a, b, jobs_a);
  const int ra = reduce_grid(a), rb = reduce_grid(b);
  gemm_reduce_pair_kernel<<<ra + rb, 256, 0, s>>>(a, b, ra, b_lo);
  return hipGetLastError();
}

// ------------------------------------------------ few rows (decode) ---
// C = A B^T for at most 64 rows of A (bf16 operands, unit k strides, the
// A1 / A2 and B1 / Bm switches at K1 as on the 256 x 256 kernel): the
// weights B stream from HBM once, split over (N / 64 column blocks) x
// nsplit K shares so that every CU holds a share. A workgroup's four waves
// own 16 columns each and all the rows (MB blocks of 16) on the 16x16x32
// MFMA, whose operand layout lets every lane read its 16 bytes of A and B
// straight from memory (no LDS); a ring of R steps (32 k each) keeps the
// loads R - 1 steps ahead of the multiplies. Shares write float32 partials
// [share][M][N] that gemm_reduce_kernel adds in order; a single share
// writes C.
constexpr int kSkinnyRows = 64, kSkinnyCols = 64, kSkinnyK = 32;

template <typename TC, int MB>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs g) {
  if (g.header && g.header[0] != 0) return;
  constexpr int R = MB == 4 ? 6 : 8;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, kg = (lane >> 4) * 8;
  const int ntiles = g.N / kSkinnyCols;
  const int nt = blockIdx.x % ntiles, kz = blockIdx.x / ntiles;
  const int col = nt * kSkinnyCols + w * 16 + r;  // this lane's B row
  const int kshare = g.K / g.nsplit, kbeg = kz * kshare;
  const int steps = kshare / kSkinnyK;
  const uint16_t* A1 = static_cast<const uint16_t*>(g.A1);
  const uint16_t* A2 = static_cast<const uint16_t*>(g.A2);
  const uint16_t* a1[MB];
  const uint16_t* a2[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = min(mb * 16 + r, g.M - 1);  // rows past M: never stored
    a1[mb] = A1 + static_cast<int64_t>(m) * g.a1_m + kg;
    a2[mb] = A2 + static_cast<int64_t>(m) * g.a2_m + kg;
  }
  const uint16_t* b1 =
      g.B1 ? static_cast<const uint16_t*>(g.B1) + col * g.b1_n + kg : nullptr;
  const uint16_t* bm = static_cast<const uint16_t*>(g.Bm) + col * g.b_n + kg;
  uint4 av[R][MB], bv[R];
  auto load = [&](int k0, uint4 (&ad)[MB], uint4& bd) {
    const bool first = k0 < g.K1;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      ad[mb] = *reinterpret_cast<const uint4*>(first ? a1[mb] + k0
                                                     : a2[mb] + (k0 - g.K1));
    bd = *reinterpret_cast<const uint4*>(
        first && b1 ? b1 + k0 : bm + (!first && g.b2_rel ? k0 - g.K1 : k0));
  };
  floatx4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < R - 1; ++q)
    if (q < steps) load(kbeg + q * kSkinnyK, av[q], bv[q]);
  for (int base = 0; base < steps; base += R) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int t = base + q;
      if (t >= steps) break;
      const int tn = t + R - 1;
      if (tn < steps)
        load(kbeg + tn * kSkinnyK, av[(q + R - 1) % R], bv[(q + R - 1) % R]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = mfma_bf16(av[q][mb], bv[q], acc[mb]);
    }
  }
  // element i of block mb: row mb*16 + 4*(lane >> 4) + i, column col
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mb * 16 + (lane >> 4) * 4 + i;
      if (m >= g.M) continue;
      if (g.nsplit > 1)
        g.part[(static_cast<int64_t>(kz) * g.M + m) * g.N + col] = acc[mb][i];
      else
        st<TC>(static_cast<TC*>(g.C), static_cast<int64_t>(m) * g.c_m + col,
               acc[mb][i]);
    }
}

static bool gemm_skinny_ok(const GemmArgs& g) {
  return g.M > 0 && g.M <= kSkinnyRows && g.N % kSkinnyCols == 0 &&
         g.K % kSkinnyK == 0 && g.K1 % kSkinnyK == 0 && g.a1_k == 1 &&
         g.a2_k == 1 && g.b_k == 1 && g.a1_m % 8 == 0 && g.a2_m % 8 == 0 &&
         g.b_n % 8 == 0 && (!g.B1 || g.b1_n % 8 == 0) && !g.ln_stats_out &&
         !g.ln_rows && !g.ln_quad_a;
}

// K shares: about two workgroups a CU (the column blocks times the
// shares) but at most 8 shares (16 made the in-order sum of the partials
// cost more than the extra workgroups saved: 23.4 against 22.0 us for
// W_mix at 64 tokens), whole 32-wide steps in every share, the partials
// within part_floats.
template <typename T>
__global__ __launch_bounds__(256) void reduce_ln_rows_kernel(LnArgs a,
                                                           const float* part,
                                                           int ns, int64_t mn);

// K shares of the few-rows kernel for g.
static int skinny_shares(const GemmArgs& g, const float* part,
                         int64_t part_floats, int cus) {
  const int ntiles = g.N / kSkinnyCols;
  const int64_t mn = static_cast<int64_t>(g.M) * g.N;
  int ns = std::max(1, std::min(8, (2 * cus + ntiles - 1) / ntiles));
  while (ns > 1 && (g.K % (ns * kSkinnyK) != 0 || !part ||
                    ns * mn > part_floats))
    --ns;
  return ns;
}

// Whether the shares' sums can go straight into the row LayerNorm: K split,
// u = A B^T is the LayerNorm input with d = N a multiple of 1024 up to 4096,
// no saved copies.
static bool skinny_ln_ok(const GemmArgs& g, const LnArgs& ln, int ns) {
  return ns > 1 && ln.d == g.N && ln.d % 1024 == 0 && ln.d <= 4096 &&
         !ln.h_save;
}

// With ln (skinny_ln_ok must hold), the shares' sums go into the row
// LayerNorm (reduce_ln_rows_kernel) instead of the reduce kernel: h in
// place of u.
static hipError_t gemm_skinny_launch(const GemmArgs& g0, int c_type,
                                     hipStream_t s, float* part,
                                     int64_t part_floats, int cus,
                                     const LnArgs* ln = nullptr) {
  GemmArgs g = g0;
  const int ntiles = g.N / kSkinnyCols;
  const int64_t mn = static_cast<int64_t>(g.M) * g.N;
  const int ns = skinny_shares(g, part, part_floats, cus);
  g.nsplit = ns;
  g.part = ns > 1 ? part : nullptr;
  const int grid = ntiles * ns;
  const bool f32 = ns > 1 || c_type != kBF16;
#define L3_SKINNY(MB)                                          \
  {                                                            \
    if (f32)                                                   \
      gemm_skinny_kernel<float, MB><<<grid, 256, 0, s>>>(g);   \
    else                                                       \
      gemm_skinny_kernel<uint16_t, MB><<<grid, 256, 0, s>>>(g); \
  }
  if (g.M <= 16)
    L3_SKINNY(1)
  else if (g.M <= 32)
    L3_SKINNY(2)
  else
    L3_SKINNY(4)
#undef L3_SKINNY
  if (ln) {
    if (c_type == kBF16)
      reduce_ln_rows_kernel<uint16_t><<<g.M, 256, 0, s>>>(*ln, part, ns, mn);
    else
      reduce_ln_rows_kernel<float><<<g.M, 256, 0, s>>>(*ln, part, ns, mn);
  } else if (ns > 1) {
    const int rgrid = reduce_grid(g);
    if (c_type == kBF16)
      gemm_reduce_kernel<uint16_t><<<rgrid, 256, 0, s>>>(g);
    else
      gemm_reduce_kernel<float><<<rgrid, 256, 0, s>>>(g);
  }
  return hipGetLastError();
}

// ------------------------------------------- LayerNorm fold into W_mix ---
// LayerNorm followed by a product, sum_k W[n, k] h[m, k] with
// h = gamma * (u - mean) * rstd + beta, equals
//   rstd * (sum_k W1[n, k] u[m, k] - mean * c1[n]) + c2[n],
//   W1[n, k] = W[n, k] gamma[k], c1[n] = sum_k W1[n, k],
//   c2[n] = sum_k W[n, k] beta[k].
// W1 is rounded to bf16 (the GEMM operand) and c1 is summed from the rounded
// values, so the mean term cancels against the rounded product exactly (up
// to float32 rounding): the error follows the deviations u - mean, not u.
// One wave per output column n, 8 elements a lane and step.
__device__ __forceinline__ void ln_fold_block(const LnFoldArgs& a, int blk) {
  if (a.header[0] != 0) return;
  const int lane = threadIdx.x & 63;
  const int n = blk * 4 + (threadIdx.x >> 6);
  if (n >= a.n) return;
  const uint16_t* w = a.W + static_cast<int64_t>(n) * a.w_n;
  uint16_t* w1 =
      a.W1 ? a.W1 + static_cast<int64_t>(n) * a.d * (a.split ? 2 : 1) : nullptr;
  float c1 = 0.f, c2 = 0.f;
  for (int e0 = lane * 8; e0 < a.d; e0 += 512) {
    const u32x4 wv = *reinterpret_cast<const u32x4*>(w + e0);
    const u32x4 gv = *reinterpret_cast<const u32x4*>(a.gamma + e0);
    const u32x4 bv = *reinterpret_cast<const u32x4*>(a.beta + e0);
    u32x4 o, lo;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float w0 = __uint_as_float(wv[q] << 16);
      const float w1v = __uint_as_float(wv[q] & 0xffff0000u);
      // products of two bf16 values are exact in float32
      const float p0 = w0 * __uint_as_float(gv[q] << 16);
      const float p1 = w1v * __uint_as_float(gv[q] & 0xffff0000u);
      o[q] = f2bf2(p0, p1);
      lo[q] = f2bf2(p0 - __uint_as_float(o[q] << 16),
                    p1 - __uint_as_float(o[q] & 0xffff0000u));
      c1 += __uint_as_float(o[q] << 16) + __uint_as_float(o[q] & 0xffff0000u);
      c2 = fmaf(w0, __uint_as_float(bv[q] << 16), c2);
      c2 = fmaf(w1v, __uint_as_float(bv[q] & 0xffff0000u), c2);
    }
    if (a.W1) {
      *reinterpret_cast<u32x4*>(w1 + e0) = o;
      if (a.split) *reinterpret_cast<u32x4*>(w1 + a.d + e0) = lo;
    }
  }
  c1 = a.split ? 0.f : wave_sum(c1);
  c2 = wave_sum(c2);
  if (lane == 0) {
    a.c12[2 * n] = c1;
    a.c12[2 * n + 1] = c2;
  }
}

__global__ __launch_bounds__(256) void ln_fold_kernel(LnFoldArgs a) {
  ln_fold_block(a, blockIdx.x);
}

hipError_t ln_fold_launch(const LnFoldArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  ln_fold_kernel<<<ceil_div(a.n, 4), 256, 0, s>>>(a);
  return hipGetLastError();
}

// Per row: Chan's combination of the nparts equal-sized (256-column)
// partial (mean, M2) pairs of the W_up epilogue: mean of the means,
// M2 = sum of the parts' M2 + 256 * sum of squared deviations of the part
// means; biased variance M2 / d; out (rstd, -mean * rstd).
__global__ __launch_bounds__(256) void ln_rows_kernel(LnRowsArgs a) {
  if (a.header[0] != 0) return;
  const int row = blockIdx.x * 256 + threadIdx.x;
  if (row >= a.B) return;
  const float2* p =
      reinterpret_cast<const float2*>(a.part) + static_cast<int64_t>(row) * a.nparts;
  if (a.quad) {
    float q2 = 0.f;
    for (int q = 0; q < a.nparts; ++q) q2 += p[q].x;
    const float rstd = 1.0f / sqrtf(fmaxf(q2, 0.f) / a.d + a.eps);
    reinterpret_cast<float2*>(a.rows)[row] = make_float2(rstd, 0.f);
    return;
  }
  float mean = 0.f;
  for (int q = 0; q < a.nparts; ++q) mean += p[q].x;
  mean /= a.nparts;
  float m2 = 0.f, dev = 0.f;
  for (int q = 0; q < a.nparts; ++q) {
    const float2 v = p[q];
    const float c = v.x - mean;
    m2 += v.y;
    dev = fmaf(c, c, dev);
  }
  m2 = fmaf(256.0f, dev, m2);
  const float rstd = 1.0f / sqrtf(m2 / a.d + a.eps);
  reinterpret_cast<float2*>(a.rows)[row] = make_float2(rstd, -mean * rstd);
}

hipError_t ln_rows_launch(const LnRowsArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  ln_rows_kernel<<<ceil_div(a.B, 256), 256, 0, s>>>(a);
  return hipGetLastError();
}

// W_up folded through LayerNorm (inference): with Wc = W - 1 mean_r(W)
// (columns centred over the d rows), u - mean(u) = Wc a, so
//   sum_j (u_j - mean)^2 = a^T (Wc^T Wc) a  and
//   W_mix1 h = rstd * (W_mix1 diag(gamma) Wc) a + W_mix1 beta,
// one d_e x d_e and one d x d_e matrix built from the weights per call.
// The centring removes the mean exactly, so neither product cancels a
// large mean against the rest. G takes Wc^T as bf16 hi | lo (3 terms on the
// bf16 kernel: hi hi + lo hi + hi lo, about float32 accuracy); the other
// takes W_mix1 as it is (bf16, exact) against (diag(gamma) Wc)^T as hi | lo
// (2 terms, the same accuracy: gamma moves to the side that is split
// anyway, and W_mix1 diag(gamma) is never formed).
// Column sums of W (rows x cols, bf16) over blocks of 64 rows:
// part[y * cols + c] = sum of W[r, c] over rows r of block y.
__device__ __forceinline__ void col_part_block(const int32_t* header,
                                               const uint16_t* W, int rows,
                                               int cols, float* part, int bx,
                                               int by) {
  if (header[0] != 0) return;
  __shared__ float s[4][64];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int c = bx * 64 + tx, r0 = by * 64;
  float acc = 0.f;
  if (c < cols) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int r = r0 + ty + 4 * k;
      if (r < rows) acc += bf2f(W[static_cast<int64_t>(r) * cols + c]);
    }
  }
  s[ty][tx] = acc;
  __syncthreads();
  if (ty == 0 && c < cols)
    part[static_cast<int64_t>(by) * cols + c] =
        (s[0][tx] + s[1][tx]) + (s[2][tx] + s[3][tx]);
}

__global__ __launch_bounds__(256) void col_part_kernel(const int32_t* header,
                                                       const uint16_t* W,
                                                       int rows, int cols,
                                                       float* part) {
  col_part_block(header, W, rows, cols, part, blockIdx.x, blockIdx.y);
}

// ln_fold's blocks (the first nfold) and col_part's (cbx column blocks a
// row block) in one launch: the two read different weights and write
// different buffers.
__global__ __launch_bounds__(256) void fold_prep_kernel(LnFoldArgs a,
                                                        const uint16_t* W,
                                                        int rows, int cols,
                                                        float* part, int nfold,
                                                        int cbx) {
  const int b = blockIdx.x;
  if (b < nfold) {
    ln_fold_block(a, b);
  } else {
    const int c = b - nfold;
    col_part_block(a.header, W, rows, cols, part, c % cbx, c / cbx);
  }
}

// T from W and the block sums above (added in block order per column);
// with T2, also T2[c, r] = hi, T2[c, rows + r] = lo of gamma[r] (W[r, c] -
// mean_r W[r, c]) (T2 is [cols x 2 rows]).
__global__ __launch_bounds__(256) void center_split_t_kernel(
    const int32_t* header, const uint16_t* W, int rows, int cols,
    const float* part, uint16_t* T, const uint16_t* gamma, uint16_t* T2) {
  if (header[0] != 0) return;
  __shared__ float t[64][65];
  __shared__ float s_mean[64];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  {
    // four phases of the block sums in parallel, then in phase order
    float m = 0.f;
    if (c0 + tx < cols)
#pragma unroll 8
      for (int y = ty; y < static_cast<int>(gridDim.y); y += 4)
        m += part[static_cast<int64_t>(y) * cols + c0 + tx];
    t[ty][tx] = m;
  }
  __syncthreads();
  if (ty == 0) s_mean[tx] = ((t[0][tx] + t[1][tx]) + (t[2][tx] + t[3][tx])) / rows;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = r0 + ty + 4 * k, c = c0 + tx;
    if (r < rows && c < cols)
      t[ty + 4 * k][tx] =
          bf2f(W[static_cast<int64_t>(r) * cols + c]) - s_mean[tx];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int c = c0 + ty + 4 * k, r = r0 + tx;
    if (r < rows && c < cols) {
      const float v = t[tx][ty + 4 * k];
      const uint16_t hi = f2bf(v);
      const float hv = __uint_as_float(static_cast<uint32_t>(hi) << 16);
      uint16_t* row = T + static_cast<int64_t>(c) * 3 * rows;
      row[r] = hi;
      row[rows + r] = hi;
      row[2 * rows + r] = f2bf(v - hv);
      if (T2) {
        const float gv = v * bf2f(gamma[r]);
        const uint16_t ghi = f2bf(gv);
        uint16_t* row2 = T2 + static_cast<int64_t>(c) * 2 * rows;
        row2[r] = ghi;
        row2[rows + r] =
            f2bf(gv - __uint_as_float(static_cast<uint32_t>(ghi) << 16));
      }
    }
  }
}

// Row-major counterpart for the bf16-u inference paths: out row r (stride
// 2 cols) = [hi | lo] of W[r, :] - column means, so that u = a W^T taken
// over K = 2 cols against (a, a) is the centred u - mean(u) to about float32
// accuracy. LayerNorm subtracts the mean anyway, so its output is unchanged,
// and u stored as bf16 then rounds relative to its spread, not its mean.
__global__ __launch_bounds__(256) void center_split_kernel(
    const int32_t* header, const uint16_t* W, int rows, int cols,
    const float* part, uint16_t* out) {
  if (header[0] != 0) return;
  __shared__ float t[4][64];
  __shared__ float s_mean[64];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  {
    float m = 0.f;
    if (c0 + tx < cols)
#pragma unroll 8
      for (int y = ty; y < static_cast<int>(gridDim.y); y += 4)
        m += part[static_cast<int64_t>(y) * cols + c0 + tx];
    t[ty][tx] = m;
  }
  __syncthreads();
  if (ty == 0) s_mean[tx] = ((t[0][tx] + t[1][tx]) + (t[2][tx] + t[3][tx])) / rows;
  __syncthreads();
  const int c = c0 + tx;
  if (c >= cols) return;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = r0 + ty + 4 * k;
    if (r < rows) {
      const float v = bf2f(W[static_cast<int64_t>(r) * cols + c]) - s_mean[tx];
      const uint16_t hi = f2bf(v);
      const float hv = __uint_as_float(static_cast<uint32_t>(hi) << 16);
      uint16_t* row = out + static_cast<int64_t>(r) * 2 * cols;
      row[c] = hi;
      row[cols + c] = f2bf(v - hv);
    }
  }
}

hipError_t center_split_launch(const int32_t* header, const uint16_t* W,
                               int rows, int cols, float* mean, uint16_t* out,
                               hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  dim3 grid(ceil_div(cols, 64), ceil_div(rows, 64));
  col_part_kernel<<<grid, 256, 0, s>>>(header, W, rows, cols, mean);
  center_split_kernel<<<grid, 256, 0, s>>>(header, W, rows, cols, mean, out);
  return hipGetLastError();
}

hipError_t center_split_t_launch(const int32_t* header, const uint16_t* W,
                                 int rows, int cols, float* mean, uint16_t* T,
                                 hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  dim3 grid(ceil_div(cols, 64), ceil_div(rows, 64));
  col_part_kernel<<<grid, 256, 0, s>>>(header, W, rows, cols, mean);
  center_split_t_kernel<<<grid, 256, 0, s>>>(header, W, rows, cols, mean, T,
                                             nullptr, nullptr);
  return hipGetLastError();
}

hipError_t fold_prep_launch(const LnFoldArgs& fa, const uint16_t* W,
                            int rows, int cols, float* mean, uint16_t* T,
                            const uint16_t* gamma, uint16_t* T2,
                            hipStream_t s) {
  if (fa.n <= 0 || rows <= 0 || cols <= 0) return hipErrorInvalidValue;
  const int nfold = ceil_div(fa.n, 4), cbx = ceil_div(cols, 64),
            cby = ceil_div(rows, 64);
  fold_prep_kernel<<<nfold + cbx * cby, 256, 0, s>>>(fa, W, rows, cols, mean,
                                                     nfold, cbx);
  center_split_t_kernel<<<dim3(cbx, cby), 256, 0, s>>>(fa.header, W, rows,
                                                       cols, mean, T, gamma,
                                                       T2);
  return hipGetLastError();
}

// The quadratic-form epilogue on 256 x 256 tiles (no K split, C unwritten).
hipError_t gemm_nt_256_quad_launch(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  if (!gemm_nt_256_shape_ok(g) || !g.ln_quad_a || !g.ln_stats_out ||
      g.ln_rows || g.nsplit != 1)
    return hipErrorInvalidValue;
  const int grid =
      static_cast<int>(static_cast<int64_t>(ceil_div(g.M, kTM)) * (g.N / kTN));
  gemm_nt_256_kernel<float, false, true><<<grid, 256, 0, s>>>(g);
  return hipGetLastError();
}

bool gemm_nt_mfma_ok(const GemmArgs& g) {
  return g.M > 0 && g.N % kBN == 0 && g.K % kBK == 0 && g.K1 % kBK == 0 &&
         g.a1_k == 1 && g.a2_k == 1 && g.b_k == 1 && g.a1_m % 8 == 0 &&
         g.a2_m % 8 == 0 && g.b_n % 8 == 0;
}

// bf16 operands, by size: at most 64 rows (decode): the few-rows kernel
// above; other shapes with few output tiles: K split over workgroups, so
// that the weights stream through every CU; else 256 x 256 tiles where
// their shape rules allow
// (faster than 128 x 128 tiles even when they do not fill the GPU: at
// 8192 x 1024 x 2048, 0.052 ms against 0.18); else 128 x 128 tiles.
hipError_t gemm_nt_mfma_launch(const GemmArgs& g, int c_type, hipStream_t s,
                               float* part, int64_t part_floats) {
  if (g.M <= 0) return hipSuccess;
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                              dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  const int64_t tiles256 =
      static_cast<int64_t>(ceil_div(g.M, kTM)) * (g.N / kTN);
  const int64_t tiles128 =
      static_cast<int64_t>(ceil_div(g.M, kBM)) * (g.N / kBN);
  if (gemm_skinny_ok(g))
    return gemm_skinny_launch(g, c_type, s, part, part_floats, cus);
  if (tiles128 < cus && part) {
    // few rows: the weights stream through every CU on the bf16 256 x 256
    // kernel with K split (rows past M read as zero), else the generic
    // kernel with K split
    if (gemm_nt_256_shape_ok(g) && !g.ln_stats_out && !g.ln_rows)
      return gemm_nt_256_splitk_launch(g, s, part, part_floats, 32, c_type);
    return gemm_launch(g, kBF16, kBF16, c_type, s, part, part_floats);
  }
  if (gemm_nt_256_ok(g)) {
    const int grid = static_cast<int>(tiles256);
    // the LayerNorm fold (consumer side) has its own instantiation
    if (c_type == kBF16 && g.ln_rows)
      gemm_nt_256_kernel<uint16_t, true><<<grid, 256, 0, s>>>(g);
    else if (c_type == kBF16 && g.ln_stats_out && !g.ln_quad_a &&
             g.nsplit == 1 && grid < cus)
      // the fold's producer with too few 256-row tiles: 128-row tiles
      gemm_nt_256w8_kernel<uint16_t, false, 2, true><<<
          static_cast<int>(static_cast<int64_t>(ceil_div(g.M, 128)) *
                           (g.N / kTN)),
          512, 0, s>>>(g);
    else if (c_type == kBF16)
      gemm_nt_256_kernel<uint16_t, false><<<grid, 256, 0, s>>>(g);
    else if (g.ln_rows && g.nsplit == 1 && !g.ln_stats_out && grid < cus)
      // too few 256-row tiles to fill the GPU: 128-row tiles
      gemm_nt_256w8_kernel<float, true, 2><<<
          static_cast<int>(static_cast<int64_t>(ceil_div(g.M, 128)) *
                           (g.N / kTN)),
          512, 0, s>>>(g);
    else if (g.ln_rows && g.nsplit == 1 && !g.ln_stats_out)
      gemm_nt_256w8_kernel<float, true, 4><<<grid, 512, 0, s>>>(g);
    else if (g.ln_rows)
      gemm_nt_256_kernel<float, true><<<grid, 256, 0, s>>>(g);
    else
      gemm_nt_256_kernel<float, false><<<grid, 256, 0, s>>>(g);
    return hipGetLastError();
  }
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

// The same with the row held in registers (d a multiple of 256, at most
// kLnRegChunks * 256): lane l loads columns 256 c + 4 l .. + 3 of every
// 256-column chunk c as one float4, all loads in flight together, then the
// mean and the biased variance in two passes over the registers, then h
// (and the saved copies). One read of u instead of three strided passes,
// whose dependent loads dominate at small batches (64 rows of d = 2048:
// 12 against 28 us).
constexpr int kLnRegChunks = 16;
template <typename T>
__global__ __launch_bounds__(256) void layernorm_rows_reg_kernel(LnArgs a) {
  if (a.header[0] != 0) return;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.B) return;
  const int nc = a.d >> 8;
  const int64_t base = static_cast<int64_t>(row) * a.d;
  const float* u = a.U + base + lane * 4;
  float4 v[kLnRegChunks];
#pragma unroll
  for (int c = 0; c < kLnRegChunks; ++c)
    v[c] = c < nc ? *reinterpret_cast<const float4*>(u + c * 256)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kLnRegChunks; ++c)
    if (c < nc) s += (v[c].x + v[c].y) + (v[c].z + v[c].w);
  const float mean = wave_sum(s) / a.d;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < kLnRegChunks; ++c)
    if (c < nc) {
      const float c0 = v[c].x - mean, c1 = v[c].y - mean, c2 = v[c].z - mean,
                  c3 = v[c].w - mean;
      q += (c0 * c0 + c1 * c1) + (c2 * c2 + c3 * c3);
    }
  const float var = wave_sum(q) / a.d;
  const float rstd = 1.0f / sqrtf(var + a.eps);
  const T* gamma = static_cast<const T*>(a.gamma);
  const T* beta = static_cast<const T*>(a.beta);
  T* h = static_cast<T*>(a.h);
#pragma unroll
  for (int c = 0; c < kLnRegChunks; ++c) {
    if (c >= nc) continue;
    const int e = c * 256 + lane * 4;
    const float vv[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float uh = (vv[k] - mean) * rstd;
      const float hv = ld<T>(gamma, e + k) * uh + ld<T>(beta, e + k);
      st<T>(h, base + e + k, hv);
      if (a.h_save) {
        a.h_save[base + e + k] = hv;
        a.uhat_save[base + e + k] = uh;
      }
    }
  }
  if (a.rstd_save && lane == 0) a.rstd_save[row] = rstd;
}

hipError_t ln_launch(const LnArgs& a, int dtype, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  const int grid = ceil_div(a.B, 4);
  // small batches (latency-bound) take the register form; at large ones
  // the strided kernel's many waves hide its load latency (65536 rows of
  // d = 2048: 0.535 against 0.559 ms)
  const bool reg =
      a.B <= 2048 && a.d % 256 == 0 && a.d <= kLnRegChunks * 256;
  if (dtype == kBF16 && reg)
    layernorm_rows_reg_kernel<uint16_t><<<grid, 256, 0, s>>>(a);
  else if (dtype == kBF16)
    layernorm_rows_kernel<uint16_t><<<grid, 256, 0, s>>>(a);
  else if (reg)
    layernorm_rows_reg_kernel<float><<<grid, 256, 0, s>>>(a);
  else
    layernorm_rows_kernel<float><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

// LayerNorm of rows whose input is the in-order sum of ns split-K partials
// (part[z * mn + row * d + col]): one workgroup a row, wave w holding
// columns w*d/4 .. as float4s of 256-column chunks (every share's loads in
// flight together), the row's sum and sum of squared deviations met in LDS
// from the four waves, then h. The shares are added in share order.
constexpr int kRedLnShares = 8;
template <typename T>
__global__ __launch_bounds__(256) void reduce_ln_rows_kernel(LnArgs a,
                                                           const float* part,
                                                           int ns,
                                                           int64_t mn) {
  if (a.header[0] != 0) return;
  __shared__ float s_red[2][4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = blockIdx.x;
  const int ncw = a.d >> 10;  // 256-column chunks a wave, 1 .. 4
  const int64_t base = static_cast<int64_t>(row) * a.d;
  const int col0 = w * (a.d >> 2) + lane * 4;
  // every load is issued unconditionally (shares past ns and chunks past
  // the row re-read share 0 / chunk 0, inside the buffer) so that they are
  // all in flight together; only the sums are predicated
  float4 v[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int cc = c < ncw ? c : 0;
    float4 q[kRedLnShares];
#pragma unroll
    for (int z = 0; z < kRedLnShares; ++z) {
      const int zz = z < ns ? z : 0;
      q[z] = *reinterpret_cast<const float4*>(part + zz * mn + base + col0 +
                                              cc * 256);
    }
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int z = 0; z < kRedLnShares; ++z)
      if (z < ns) {
        acc.x += q[z].x;
        acc.y += q[z].y;
        acc.z += q[z].z;
        acc.w += q[z].w;
      }
    v[c] = c < ncw ? acc : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float sm = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (c < ncw) sm += (v[c].x + v[c].y) + (v[c].z + v[c].w);
  sm = wave_sum(sm);
  if (lane == 0) s_red[0][w] = sm;
  __syncthreads();
  const float mean =
      ((s_red[0][0] + s_red[0][1]) + (s_red[0][2] + s_red[0][3])) / a.d;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (c < ncw) {
      const float c0 = v[c].x - mean, c1 = v[c].y - mean, c2 = v[c].z - mean,
                  c3 = v[c].w - mean;
      q += (c0 * c0 + c1 * c1) + (c2 * c2 + c3 * c3);
    }
  q = wave_sum(q);
  if (lane == 0) s_red[1][w] = q;
  __syncthreads();
  const float var =
      ((s_red[1][0] + s_red[1][1]) + (s_red[1][2] + s_red[1][3])) / a.d;
  const float rstd = 1.0f / sqrtf(var + a.eps);
  const T* gamma = static_cast<const T*>(a.gamma);
  const T* beta = static_cast<const T*>(a.beta);
  T* h = static_cast<T*>(a.h);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (c >= ncw) continue;
    const int e = col0 + c * 256;
    const float vv[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float uh = (vv[k] - mean) * rstd;
      st<T>(h, base + e + k, ld<T>(gamma, e + k) * uh + ld<T>(beta, e + k));
    }
  }
}

// u = A B^T in float32, then LayerNorm of each row of u into ln.h (ln.U =
// the GEMM's C). Few rows with K split: the shares' sum and the LayerNorm
// in one kernel; otherwise the GEMM and the row pass.
hipError_t gemm_ln_launch(const GemmArgs& g, const LnArgs& ln, int dtype,
                          hipStream_t s, float* part, int64_t part_floats) {
  if (g.M <= 0) return hipSuccess;
  if (gemm_skinny_ok(g)) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                              dev) != hipSuccess || cus <= 0)
      cus = 256;
    if (skinny_ln_ok(g, ln, skinny_shares(g, part, part_floats, cus)))
      return gemm_skinny_launch(g, dtype, s, part, part_floats, cus, &ln);
  }
  hipError_t e = gemm_nt_mfma_launch(g, kF32, s, part, part_floats);
  if (e == hipSuccess) e = ln_launch(ln, dtype, s);
  return e;
}

}  // namespace l3
