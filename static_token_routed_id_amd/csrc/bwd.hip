// Backward pass of the layer (the chain rule of the forward formula of the
// gist.science explainer of "L^3: Large Lookup Layers", Technical Summary,
// Core Architecture, Mathematical Formulation; the pages print no
// gradients). The projections' gradients run through the GEMM kernels;
// this file holds the LayerNorm backward, the per-id segment backward and a
// bf16 transpose for the GEMMs' operands.
//
// Determinism: nothing here uses floating-point atomics. LayerNorm column
// sums (dgamma, dbeta) are taken by one thread per column over the rows in
// order. In the segment backward every element of dK, dV has one writer
// that sums the id's tokens in sorted order, and every dx row one writer
// (Systems-Friendly Design, Batch Sorting: the sorted batch makes the mask
// block-diagonal, so ids never share rows and tokens never share ids).

#include "l3_device.h"
#include "l3_internal.h"
#include "seg_wave.h"

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

// dst[c * rows + r] = src[r * ld + c] for bf16 (the transposed copy that puts
// a product's reduction index last in both operands, as the bf16 MFMA GEMM
// reads them): 64 x 64 tiles through LDS (rows padded by two elements), each
// thread moving 16 elements; partial edge tiles are bounds-checked.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(
    const int32_t* header, const uint16_t* src, int64_t ld, int rows,
    int cols, uint16_t* dst, int64_t ldd) {
  if (header[0] != 0) return;
  __shared__ uint16_t t[64][66];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = r0 + ty + 4 * k, c = c0 + tx;
    if (r < rows && c < cols) t[ty + 4 * k][tx] = src[r * ld + c];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int c = c0 + ty + 4 * k, r = r0 + tx;
    if (r < rows && c < cols)
      dst[static_cast<int64_t>(c) * ldd + r] = t[tx][ty + 4 * k];
  }
}

hipError_t transpose_bf16_launch(const int32_t* header, const uint16_t* src,
                                 int64_t ld, int rows, int cols,
                                 uint16_t* dst, hipStream_t s, int64_t ldd) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  dim3 grid((cols + 63) / 64, (rows + 63) / 64);
  transpose_bf16_kernel<<<grid, 256, 0, s>>>(header, src, ld, rows, cols,
                                              dst, ldd > 0 ? ldd : rows);
  return hipGetLastError();
}

// Float32 [n] to bf16 hi = bf16(v), lo = bf16(v - hi) (hi + lo carries v
// to about 2^-17 relative), four elements a thread.
__global__ __launch_bounds__(256) void split_bf16_kernel(
    const int32_t* header, const float* src, int64_t n, uint16_t* hi,
    uint16_t* lo) {
  if (header[0] != 0) return;
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  if (i + 4 <= n) {
    const float4 v = *reinterpret_cast<const float4*>(src + i);
    const float vv[4] = {v.x, v.y, v.z, v.w};
    uint16_t h[4], l[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      h[q] = f2bf(vv[q]);
      l[q] = f2bf(vv[q] - __uint_as_float(static_cast<uint32_t>(h[q]) << 16));
    }
    *reinterpret_cast<uint2*>(hi + i) =
        make_uint2(h[0] | (static_cast<uint32_t>(h[1]) << 16),
                   h[2] | (static_cast<uint32_t>(h[3]) << 16));
    *reinterpret_cast<uint2*>(lo + i) =
        make_uint2(l[0] | (static_cast<uint32_t>(l[1]) << 16),
                   l[2] | (static_cast<uint32_t>(l[3]) << 16));
  } else {
    for (int64_t j = i; j < n; ++j) {
      hi[j] = f2bf(src[j]);
      lo[j] = f2bf(src[j] - __uint_as_float(static_cast<uint32_t>(hi[j]) << 16));
    }
  }
}

hipError_t split_bf16_launch(const int32_t* header, const float* src,
                             int64_t n, uint16_t* hi, uint16_t* lo,
                             hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 1023) / 1024;
  split_bf16_kernel<<<static_cast<int>(blocks), 256, 0, s>>>(header, src, n,
                                                             hi, lo);
  return hipGetLastError();
}

// Float32 src [rows x cols] (row stride ld) to its transpose in bf16 hi and
// lo halves: dst row c (stride ldd) holds hi = bf16(src[r][c]) at r, lo =
// bf16(src[r][c] - hi) at lo_off + r, and hi again at hi2_off + r if
// hi2_off >= 0. hi + lo carries src to about 2^-17 relative, so one bf16
// GEMM over the lengthened reduction (the other operand laid out to match)
// reproduces a float32 operand's product.
__global__ __launch_bounds__(256) void transpose_split_kernel(
    const int32_t* header, const float* src, int64_t ld, int rows, int cols,
    uint16_t* dst, int64_t ldd, int64_t lo_off, int64_t hi2_off) {
  if (header[0] != 0) return;
  __shared__ float t[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = r0 + ty + 4 * k, c = c0 + tx;
    if (r < rows && c < cols) t[ty + 4 * k][tx] = src[r * ld + c];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int c = c0 + ty + 4 * k, r = r0 + tx;
    if (r < rows && c < cols) {
      const float v = t[tx][ty + 4 * k];
      const uint16_t hi = f2bf(v);
      const float hv = __uint_as_float(static_cast<uint32_t>(hi) << 16);
      uint16_t* row = dst + static_cast<int64_t>(c) * ldd;
      row[r] = hi;
      row[lo_off + r] = f2bf(v - hv);
      if (hi2_off >= 0) row[hi2_off + r] = hi;
    }
  }
}

hipError_t transpose_split_launch(const int32_t* header, const float* src,
                                  int64_t ld, int rows, int cols,
                                  uint16_t* dst, hipStream_t s, int64_t ldd,
                                  int64_t lo_off, int64_t hi2_off) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  dim3 grid((cols + 63) / 64, (rows + 63) / 64);
  transpose_split_kernel<<<grid, 256, 0, s>>>(
      header, src, ld, rows, cols, dst, ldd > 0 ? ldd : 2 * int64_t(rows),
      lo_off > 0 ? lo_off : rows, hi2_off);
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

// dgamma[j] = sum_i dh[i, j] * uhat[i, j], dbeta[j] = sum_i dh[i, j], in a
// fixed order: each workgroup sums a block of 256 rows for 64 columns (four
// row phases of 64 rows, combined in order), then one thread per column
// adds the blocks in order.
constexpr int kLnRowBlk = 256;

__global__ __launch_bounds__(256) void ln_bwd_cols_kernel(BwdArgs a) {
  __shared__ float s_g[4][64], s_b[4][64];
  if (a.header[0] != 0) return;
  const int c = threadIdx.x & 63, ph = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + c;
  const int rb = blockIdx.y;
  float sg = 0.f, sb = 0.f;
  if (j < a.d) {
    const int i0 = rb * kLnRowBlk + ph * 64;
    const int i1 = min(i0 + 64, a.B);
    for (int i = i0; i < i1; ++i) {
      const int64_t o = static_cast<int64_t>(i) * a.d + j;
      sg = fmaf(a.dH[o], a.uhat[o], sg);
      sb += a.dH[o];
    }
  }
  s_g[ph][c] = sg;
  s_b[ph][c] = sb;
  __syncthreads();
  if (ph == 0 && j < a.d) {
    const int64_t o = (static_cast<int64_t>(rb) * 2) * a.d + j;
    a.ln_part[o] = ((s_g[0][c] + s_g[1][c]) + s_g[2][c]) + s_g[3][c];
    a.ln_part[o + a.d] = ((s_b[0][c] + s_b[1][c]) + s_b[2][c]) + s_b[3][c];
  }
}

__global__ __launch_bounds__(256) void ln_bwd_cols_sum_kernel(BwdArgs a,
                                                              int nrb) {
  if (a.header[0] != 0) return;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= a.d) return;
  float sg = 0.f, sb = 0.f;
  for (int rb = 0; rb < nrb; ++rb) {
    const int64_t o = (static_cast<int64_t>(rb) * 2) * a.d + j;
    sg += a.ln_part[o];
    sb += a.ln_part[o + a.d];
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
    const int nrb = ceil_div(a.B, kLnRowBlk);
    ln_bwd_cols_kernel<<<dim3(ceil_div(a.d, 64), nrb), 256, 0, s>>>(a);
    ln_bwd_cols_sum_kernel<<<ceil_div(a.d, 256), 256, 0, s>>>(a, nrb);
  } else {
    ln_bwd_cols_sum_kernel<<<ceil_div(a.d, 256), 256, 0, s>>>(a, 0);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------- segment bwd ---
// Two passes, both over the id-sorted batch, neither with atomics:
//
// Tiles (one wavefront per tile of <= 16 tokens of one id, all n <= k_max
// of its rows, the training forward's own work items): recompute the
// scores S = X K_t^T (the forward's MFMA code) and dP = dA V_t^T (16x16x4
// float32 MFMA), both as float32, in row chunks of 128; then per token the
// exact softmax p, dS = p * (dP - p . dP); p and dS go to two
// [B x k] float32 scratch arrays (token in sorted order, row j); finally
// dX_att = dS K_t, added to the token's dx row (each token belongs to one
// tile, so it has one writer).
//
// Rows (one workgroup per (id, block of 64 rows, block of 256 columns of
// [K | V])): dK_t[j, c] = sum_i dS[i, j] x_i[c] and dV_t[j, c] =
// sum_i p[i, j] dA_i[c] over the id's tokens in sorted order, one thread
// per column with the 64 rows in registers; each table element has exactly
// one writer, which stores the whole sum.

constexpr int kBwdRowBlk = 64;
constexpr int kBwdColBlk = 256;

// Per-token softmax statistics of one tile, merged over row chunks: running
// max M, L = sum_j exp(S_j - M), Q = sum_j exp(S_j - M) dP_j. Lane group g
// holds tokens 4g .. 4g + 3 (element i); all 16 lanes of a group agree.
struct TileStats {
  float M[4], L[4], Q[4];
};

// Scores and dP of rows c0 .. c0 + nc - 1 of one tile: the raw values go to
// the p / dS arrays (each lane writes, and later rereads, only its own
// entries) and the chunk is folded into the statistics.
template <typename T, int NB>
__device__ __forceinline__ void bwd_chunk(const BwdArgs& a, const T* xr,
                                          const float* dar, int64_t rowbase,
                                          int nc, int r, int g, int pbase,
                                          int c0, int mcount, TileStats& st) {
  floatx4 sacc[kNBMax], dacc[kNBMax];
  const T* kt = static_cast<const T*>(a.K) + rowbase * a.d;
  if constexpr (sizeof(T) == 2) {
    constexpr int R = NB == 1 ? 8 : (NB == 2 ? 4 : 2);
    if (R > 2 && (a.d / 32) % R == 0)
      scores_bf16<NB, R>(xr, kt, a.d, nc, r, g, 0, sacc);
    else
      scores_bf16<NB, 2>(xr, kt, a.d, nc, r, g, 0, sacc);
  } else {
    scores_f32<NB>(xr, kt, a.d, nc, r, g, sacc);
  }
  // dP = dA V^T on 16x16x4 float32 MFMA, 16 columns of d_e a step (lane
  // group g supplies columns 4g .. 4g + 3, one MFMA per element)
  const T* vt = static_cast<const T*>(a.V) + rowbase * a.d_e;
  int voff[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    dacc[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    voff[nb] = min(nb * 16 + r, nc - 1) * a.d_e + g * 4;
  }
  for (int kc = 0; kc < a.d_e; kc += 16) {
    const float4 dv = *reinterpret_cast<const float4*>(dar + kc + g * 4);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float vv[4];
      if constexpr (sizeof(T) == 2) {
        const uint2 u = *reinterpret_cast<const uint2*>(vt + voff[nb] + kc);
        vv[0] = __uint_as_float(u.x << 16);
        vv[1] = __uint_as_float(u.x & 0xffff0000u);
        vv[2] = __uint_as_float(u.y << 16);
        vv[3] = __uint_as_float(u.y & 0xffff0000u);
      } else {
        const float4 f = *reinterpret_cast<const float4*>(vt + voff[nb] + kc);
        vv[0] = f.x;
        vv[1] = f.y;
        vv[2] = f.z;
        vv[3] = f.w;
      }
      dacc[nb] = mfma_f32(dv.x, vv[0], dacc[nb]);
      dacc[nb] = mfma_f32(dv.y, vv[1], dacc[nb]);
      dacc[nb] = mfma_f32(dv.z, vv[2], dacc[nb]);
      dacc[nb] = mfma_f32(dv.w, vv[3], dacc[nb]);
    }
  }
  // lane holds (token 4g + i, row c0 + nb * 16 + r)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 4 * g + i;
    float cm = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      if (nb * 16 + r < nc) cm = fmaxf(cm, sacc[nb][i]);
    cm = group16_max(cm);
    const float m_new = fmaxf(st.M[i], cm);
    float l = 0.f, q = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int j = nb * 16 + r;
      if (j < nc) {
        const float e = __expf(sacc[nb][i] - m_new);
        l += e;
        q = fmaf(e, dacc[nb][i], q);
        if (t < mcount) {
          const int64_t o = static_cast<int64_t>(pbase + t) * a.kst + c0 + j;
          a.Pbuf[o] = sacc[nb][i];
          a.DSbuf[o] = dacc[nb][i];
        }
      }
    }
    l = group16_sum(l);
    q = group16_sum(q);
    const float sc = __expf(st.M[i] - m_new);  // 0 on the first chunk
    st.L[i] = fmaf(st.L[i], sc, l);
    st.Q[i] = fmaf(st.Q[i], sc, q);
    st.M[i] = m_new;
  }
}

// Second sweep over the same lane's entries: p = exp(S - M) / L,
// dS = p * (dP - Q / L).
template <int NB>
__device__ __forceinline__ void bwd_chunk_finish(const BwdArgs& a, int nc,
                                                 int r, int g, int pbase,
                                                 int c0, int mcount,
                                                 const TileStats& st) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 4 * g + i;
    if (t < mcount) {
      const float inv = 1.0f / st.L[i];
      const float pd = st.Q[i] * inv;
      float sv[NB], dv[NB];
      const int64_t base = static_cast<int64_t>(pbase + t) * a.kst + c0 + r;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (nb * 16 + r < nc) {
          sv[nb] = a.Pbuf[base + nb * 16];
          dv[nb] = a.DSbuf[base + nb * 16];
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (nb * 16 + r < nc) {
          const float p = __expf(sv[nb] - st.M[i]) * inv;
          a.Pbuf[base + nb * 16] = p;
          a.DSbuf[base + nb * 16] = p * (dv[nb] - pd);
        }
      }
    }
  }
}

// K rows j0 .. j0 + 15 of this lane's 4 columns (c) and the 16 tokens' dS of
// those rows (one float4 per lane: token lane >> 2, rows 4 (lane & 3) ..)
template <typename T>
struct DxBlock {
  uint32_t k[16][sizeof(T) == 2 ? 2 : 4];
  float4 ds;
};

template <typename T>
__device__ __forceinline__ void dx_block_load(const BwdArgs& a, int64_t r0,
                                              int n, int j0, int c,
                                              bool active, int lane, int tok0,
                                              int mcount, DxBlock<T>& b) {
  const T* K = static_cast<const T*>(a.K);
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const int j = min(j0 + jj, n - 1);
    if (active) {
      const int64_t o = (r0 + j) * a.d + c;
      if constexpr (sizeof(T) == 2) {
        const uint2 u = *reinterpret_cast<const uint2*>(K + o);
        b.k[jj][0] = u.x;
        b.k[jj][1] = u.y;
      } else {
        const u32x4 u = *reinterpret_cast<const u32x4*>(K + o);
#pragma unroll
        for (int q = 0; q < 4; ++q) b.k[jj][q] = u[q];
      }
    }
  }
  const int t = lane >> 2, jq = (lane & 3) * 4;
  b.ds = float4{0.f, 0.f, 0.f, 0.f};
  if (t < mcount)
    b.ds = *reinterpret_cast<const float4*>(
        a.DSbuf + static_cast<int64_t>(tok0 + t) * a.kst + j0 + jq);
}

typedef short bwd_v4i16 __attribute__((ext_vector_type(4)));
constexpr int kDxS = 64 + 8;  // dX_att staging row stride (elements)

// dX_att = dS K_t (bf16 K, d a multiple of 128) on 16x16x32 bf16 MFMA, the
// same product shape as the forward's P V_t: tokens are the rows of A (dS,
// float32, entering as bf16 hi + lo halves, two MFMAs), K_t's rows the
// reduction. MB blocks of 16 tokens share every K block (MB = 4: a 64-token
// tile of a busy id reads K_t once where four 16-token tiles read it four
// times). Columns in passes of CW (CW / 16 accumulators of 16 x 16 per token
// block); K_t in blocks of 32 rows x CW columns, double buffered in
// registers a block at a time: each iteration first requests the next block
// (and its dS), then moves the current one through a wave-private LDS
// buffer, 64 columns at a time (8 lanes a 128-byte row slice), and reads it
// back as the B operand with the transposing LDS read. (A ring of single
// 64-column steps carried across iterations lost its depth to the waits the
// compiler places after a loop's back edge.) Rows past n have zero weights
// (their K rows are clamped to row n-1). Each output element sums the row
// blocks in order whatever MB and CW are.
template <int MB, int CW>
__device__ __forceinline__ void dx_att_mfma(const BwdArgs& a, int64_t r0,
                                            int n, int tok0, int mcount,
                                            int lane, uint16_t* stg,
                                            int c_begin, int c_end) {
  constexpr int SB = CW / 64;  // 64-column halves of a block
  constexpr int NB = CW / 16;  // 16-column output blocks of a pass
  const int r = lane & 15, g = lane >> 4;
  const uint16_t* K = static_cast<const uint16_t*>(a.K);
  const int trow = 8 * g + (r >> 2), tcol = 4 * (r & 3);
  const int srow = lane >> 3, scol = (lane & 7) * 8;
  const int nrb = ceil_div(n, 32);
  bool tok_ok[MB];
  const float* dsr[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int t = mb * 16 + r;
    tok_ok[mb] = t < mcount;
    dsr[mb] = a.DSbuf + static_cast<int64_t>(tok0 + min(t, mcount - 1)) * a.kst;
  }
  auto ds_load = [&](int rb, float4 (&v0)[MB], float4 (&v1)[MB]) {
    const int j = min(rb, nrb - 1) * 32 + 8 * g;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      v0[mb] = *reinterpret_cast<const float4*>(dsr[mb] + j);
      v1[mb] = *reinterpret_cast<const float4*>(dsr[mb] + j + 4);
    }
  };
  auto split = [&](int rb, const float4& v0, const float4& v1, bool ok,
                   u32x4& hi, u32x4& lo) {
    const int j0 = rb * 32 + 8 * g;
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = ok && j0 + 2 * e < n ? v[2 * e] : 0.f;
      const float x1 = ok && j0 + 2 * e + 1 < n ? v[2 * e + 1] : 0.f;
      h[e] = f2bf2(x0, x1);
      l[e] = f2bf2(x0 - __uint_as_float(h[e] << 16),
                   x1 - __uint_as_float(h[e] & 0xffff0000u));
    }
    hi = u32x4{h[0], h[1], h[2], h[3]};
    lo = u32x4{l[0], l[1], l[2], l[3]};
  };
  for (int cc = c_begin; cc < c_end; cc += CW) {
    // block rb: rows rb*32 .., columns cc .. cc+CW-1: chunk (sb, k) of
    // 64-column half sb, rows k*8 + srow, 8 columns at scol
    auto load_blk = [&](u32x4 (&b)[SB * 4], int rb) {
      const int j0 = min(rb, nrb - 1) * 32;
#pragma unroll
      for (int sb = 0; sb < SB; ++sb)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int j = min(j0 + k * 8 + srow, n - 1);
          b[sb * 4 + k] = *reinterpret_cast<const u32x4*>(
              K + (r0 + j) * a.d + cc + sb * 64 + scol);
        }
    };
    floatx4 acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    // block rb's dS as the A operand, its K rows through LDS as B
    auto consume = [&](const u32x4 (&b)[SB * 4], int rb,
                       const float4 (&v0)[MB], const float4 (&v1)[MB]) {
      u32x4 ahi[MB], alo[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        split(rb, v0[mb], v1[mb], tok_ok[mb], ahi[mb], alo[mb]);
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int k = 0; k < 4; ++k)
          *reinterpret_cast<u32x4*>(&stg[(k * 8 + srow) * kDxS + scol]) =
              b[sb * 4 + k];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          typedef __attribute__((address_space(3))) bwd_v4i16 lds_v4i16;
          const bwd_v4i16 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)(&stg[trow * kDxS + nb * 16 + tcol]));
          const bwd_v4i16 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)(&stg[(trow + 4) * kDxS + nb * 16 + tcol]));
          const uint2 l2 = __builtin_bit_cast(uint2, lo4);
          const uint2 h2 = __builtin_bit_cast(uint2, hi4);
          const u32x4 bf = u32x4{l2.x, l2.y, h2.x, h2.y};
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            floatx4& ac = acc[mb][sb * 4 + nb];
            ac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, ahi[mb]),
                __builtin_bit_cast(bf16x8_t, bf), ac, 0, 0, 0);
            ac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, alo[mb]),
                __builtin_bit_cast(bf16x8_t, bf), ac, 0, 0, 0);
          }
        }
      }
    };
    // two named buffers, two blocks an iteration: the block being used was
    // requested one block earlier, and nothing is copied between buffers
    u32x4 bA[SB * 4], bB[SB * 4];
    float4 dA0[MB], dA1[MB], dB0[MB], dB1[MB];
    ds_load(0, dA0, dA1);
    load_blk(bA, 0);
    for (int rb = 0; rb < nrb; rb += 2) {
      ds_load(rb + 1, dB0, dB1);
      load_blk(bB, rb + 1);
      consume(bA, rb, dA0, dA1);
      if (rb + 1 < nrb) {
        ds_load(rb + 2, dA0, dA1);
        load_blk(bA, rb + 2);
        consume(bB, rb + 1, dB0, dB1);
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = mb * 16 + 4 * g + i;
        if (t < mcount) {
          float* dst =
              a.dx + static_cast<int64_t>(a.perm[tok0 + t]) * a.d + cc + r;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) dst[nb * 16] += acc[mb][nb][i];
        }
      }
  }
}

template <typename T>
__device__ __forceinline__ void bwd_tile(const BwdArgs& a, int s, int tile,
                                         int lane, float* lds) {
  const int r = lane & 15, g = lane >> 4;
  const int t_begin = a.seg_tok_start[s];
  const int m = a.seg_tok_start[s + 1] - t_begin;
  const int n = a.seg_n[s];
  const int64_t r0 = a.seg_row_off[s];
  const int tok0 = t_begin + tile * kTokTile;
  const int mcount = min(kTokTile, m - tile * kTokTile);
  const int64_t xi = a.perm[tok0 + min(r, mcount - 1)];
  const T* xr = static_cast<const T*>(a.x) + xi * a.d;
  const float* dar = a.dA + xi * a.d_e;
  TileStats st;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    st.M[i] = -INFINITY;
    st.L[i] = 0.f;
    st.Q[i] = 0.f;
  }
#define L3_NB_DISPATCH(CALL)  \
  if (nbc <= 1) {             \
    CALL(1);                  \
  } else if (nbc <= 2) {      \
    CALL(2);                  \
  } else if (nbc <= 4) {      \
    CALL(4);                  \
  } else {                    \
    CALL(8);                  \
  }
  for (int c0 = 0; c0 < n; c0 += kWaveMaxRows) {
    const int nc = min(kWaveMaxRows, n - c0);
    const int nbc = ceil_div(nc, 16);
#define L3_CHUNK(NB) \
  bwd_chunk<T, NB>(a, xr, dar, r0 + c0, nc, r, g, tok0, c0, mcount, st)
    L3_NB_DISPATCH(L3_CHUNK)
#undef L3_CHUNK
  }
  for (int c0 = 0; c0 < n; c0 += kWaveMaxRows) {
    const int nc = min(kWaveMaxRows, n - c0);
    const int nbc = ceil_div(nc, 16);
#define L3_FIN(NB) bwd_chunk_finish<NB>(a, nc, r, g, tok0, c0, mcount, st)
    L3_NB_DISPATCH(L3_FIN)
#undef L3_FIN
  }
#undef L3_NB_DISPATCH
  // dS was written by other lanes of this wave
  __threadfence_block();
  // bf16, d a multiple of 128: dX_att is seg_bwd_dx_kernel's, one wave per
  // (tile, 128 columns), so that a busy id's tiles do not each stream all of
  // K_t through one wave
  if constexpr (sizeof(T) == 2) {
    if (a.d % 128 == 0) return;
  }
  // dX_att = dS K_t: lane owns 4 columns of a 256-column pass, all 16
  // tokens; per 16-row block the tokens' dS are staged transposed in this
  // wave's LDS ([row][token]: 4 broadcast reads a row), the next block's K
  // rows and dS already in flight while the current one is used
  for (int cc = 0; cc < a.d; cc += 256) {
    const int c = cc + lane * 4;
    const bool active = c < a.d;
    float acc[kTokTile][4];
#pragma unroll
    for (int t = 0; t < kTokTile; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[t][q] = 0.f;
    DxBlock<T> cur, nxt;
    dx_block_load<T>(a, r0, n, 0, c, active, lane, tok0, mcount, cur);
    for (int j0 = 0; j0 < n; j0 += 16) {
      if (j0 + 16 < n)
        dx_block_load<T>(a, r0, n, j0 + 16, c, active, lane, tok0, mcount,
                         nxt);
      {
        const int t = lane >> 2, jq = (lane & 3) * 4;
        const float v[4] = {cur.ds.x, cur.ds.y, cur.ds.z, cur.ds.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          lds[(jq + q) * kTokTile + t] = j0 + jq + q < n ? v[q] : 0.f;
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        float kv[4];
        if constexpr (sizeof(T) == 2) {
          kv[0] = __uint_as_float(cur.k[jj][0] << 16);
          kv[1] = __uint_as_float(cur.k[jj][0] & 0xffff0000u);
          kv[2] = __uint_as_float(cur.k[jj][1] << 16);
          kv[3] = __uint_as_float(cur.k[jj][1] & 0xffff0000u);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) kv[q] = __uint_as_float(cur.k[jj][q]);
        }
        // rows past n have zero weights
        const float4* w4 = reinterpret_cast<const float4*>(lds + jj * kTokTile);
#pragma unroll
        for (int tq = 0; tq < 4; ++tq) {
          const float4 wv = w4[tq];
          const float wt[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[tq * 4 + u][q] = fmaf(wt[u], kv[q], acc[tq * 4 + u][q]);
        }
      }
      __builtin_amdgcn_wave_barrier();
      cur = nxt;
    }
    if (active) {
#pragma unroll
      for (int t = 0; t < kTokTile; ++t) {
        if (t < mcount) {
          float* dst = a.dx + static_cast<int64_t>(a.perm[tok0 + t]) * a.d + c;
#pragma unroll
          for (int q = 0; q < 4; ++q) dst[q] += acc[t][q];
        }
      }
    }
  }
}

// The tile pass split by row chunk (bf16, d a multiple of 128): every work
// item (token tile, row chunk) of the saving forward is a wave of its own.
// seg_bwd_chunk_kernel: scores and dP of the chunk (raw, into the p / dS
// arrays) and the chunk's own softmax statistics per token (M, L, Q of its
// rows) into a [B x chunks] array; seg_bwd_finish_kernel: the tile's chunk
// statistics combined in chunk order (M = max M_c, L = sum L_c e^(M_c - M),
// Q likewise), then p and dS of the chunk. A busy id's tile so spreads over
// as many waves as it has chunks.
template <typename T>
__device__ __forceinline__ void chunk_item(const BwdArgs& a, int2 im,
                                           int lane, bool finish) {
  const int r = lane & 15, g = lane >> 4;
  const int s = im.x;
  const int n = a.seg_n[s];
  const int nch = ceil_div(n, a.chunk_rows);
  const int tile = im.y / nch, ch = im.y - tile * nch;
  const int t_begin = a.seg_tok_start[s];
  const int m = a.seg_tok_start[s + 1] - t_begin;
  const int64_t r0 = a.seg_row_off[s];
  const int tok0 = t_begin + tile * kTokTile;
  const int mcount = min(kTokTile, m - tile * kTokTile);
  const int c_lo = ch * a.chunk_rows, c_hi = min(n, c_lo + a.chunk_rows);
#define L3_NB_DISPATCH(CALL)  \
  if (nbc <= 1) {             \
    CALL(1);                  \
  } else if (nbc <= 2) {      \
    CALL(2);                  \
  } else if (nbc <= 4) {      \
    CALL(4);                  \
  } else {                    \
    CALL(8);                  \
  }
  TileStats st;
  if (!finish) {
    const int64_t xi = a.perm[tok0 + min(r, mcount - 1)];
    const T* xr = static_cast<const T*>(a.x) + xi * a.d;
    const float* dar = a.dA + xi * a.d_e;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st.M[i] = -INFINITY;
      st.L[i] = 0.f;
      st.Q[i] = 0.f;
    }
    for (int c0 = c_lo; c0 < c_hi; c0 += kWaveMaxRows) {
      const int nc = min(kWaveMaxRows, c_hi - c0);
      const int nbc = ceil_div(nc, 16);
#define L3_CHUNK(NB) \
  bwd_chunk<T, NB>(a, xr, dar, r0 + c0, nc, r, g, tok0, c0, mcount, st)
      L3_NB_DISPATCH(L3_CHUNK)
#undef L3_CHUNK
    }
    if (r == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * g + i;
        if (t < mcount)
          a.chunk_stats[static_cast<int64_t>(tok0 + t) * a.cs_stride + ch] =
              make_float4(st.M[i], st.L[i], st.Q[i], 0.f);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = min(4 * g + i, mcount - 1);
      const float4* cs = a.chunk_stats + static_cast<int64_t>(tok0 + t) * a.cs_stride;
      float M = -INFINITY;
      for (int c = 0; c < nch; ++c) M = fmaxf(M, cs[c].x);
      float L = 0.f, Q = 0.f;
      for (int c = 0; c < nch; ++c) {
        const float4 v = cs[c];
        const float sc = __expf(v.x - M);
        L = fmaf(v.y, sc, L);
        Q = fmaf(v.z, sc, Q);
      }
      st.M[i] = M;
      st.L[i] = L;
      st.Q[i] = Q;
    }
    for (int c0 = c_lo; c0 < c_hi; c0 += kWaveMaxRows) {
      const int nc = min(kWaveMaxRows, c_hi - c0);
      const int nbc = ceil_div(nc, 16);
#define L3_FIN(NB) bwd_chunk_finish<NB>(a, nc, r, g, tok0, c0, mcount, st)
      L3_NB_DISPATCH(L3_FIN)
#undef L3_FIN
    }
  }
#undef L3_NB_DISPATCH
}

template <typename T, bool FINISH>
__global__ __launch_bounds__(256, 2) void seg_bwd_chunk_kernel(BwdArgs a) {
  if (a.header[0] != 0) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n_items = a.header[a.count_slot];
  for (int item = blockIdx.x * 4 + w; item < n_items; item += gridDim.x * 4)
    chunk_item<T>(a, a.item_map[item], lane, FINISH);
}

// dX_att of the tiles, after seg_bwd_tile_kernel has written their dS: one
// wave per (tile, column pass). Ids with at least group_min_rows rows (when
// the plan made group items for them: one item of their <= 64 tokens, or
// items of 128 tokens) come first, one wave per (64 tokens of an item, 64
// columns): the 16-token blocks share every K block, so K_t is read once
// per 64 tokens. The other ids follow as the forward's work
// items (16-token tiles) with 128-column passes, the passes innermost (a
// busy id's tiles and passes spread over waves).
__global__ __launch_bounds__(256, 2) void seg_bwd_dx_kernel(BwdArgs a) {
  __shared__ __align__(16) uint16_t s_stg[4][32 * kDxS];
  if (a.header[0] != 0) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n_items = a.header[a.count_slot];
  const bool grouped = a.group_min_rows > 0 && a.gitem_map != nullptr;
  const int n_group = grouped ? a.header[3] : 0;
  const int gpass = a.d / 64;
  // two 64-token halves per group item (the second is empty for items of
  // at most 64 tokens)
  const int64_t total_g = static_cast<int64_t>(n_group) * 2 * gpass;
  const int npass = a.d / 128;
  const int64_t total = total_g + static_cast<int64_t>(n_items) * npass;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * 4 + w; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * 4) {
    if (idx < total_g) {
      const int2 im = a.gitem_map[idx / (2 * gpass)];
      const int rem = static_cast<int>(idx % (2 * gpass));
      const int half = rem / gpass, pass = rem % gpass;
      const int s = im.x;
      const int t_begin = a.seg_tok_start[s];
      const int m = a.seg_tok_start[s + 1] - t_begin;
      const int item_tok = m > kGroupTok ? kHotTok : kGroupTok;
      const int first = im.y * item_tok + half * kGroupTok;
      if (half * kGroupTok >= item_tok || first >= m) continue;
      const int tok0 = t_begin + first;
      const int mcount = min(kGroupTok, m - first);
      const int n = a.seg_n[s];
      const int64_t r0 = a.seg_row_off[s];
      if (mcount <= 16)
        dx_att_mfma<1, 64>(a, r0, n, tok0, mcount, lane, s_stg[w],
                           pass * 64, pass * 64 + 64);
      else if (mcount <= 32)
        dx_att_mfma<2, 64>(a, r0, n, tok0, mcount, lane, s_stg[w],
                           pass * 64, pass * 64 + 64);
      else
        dx_att_mfma<4, 64>(a, r0, n, tok0, mcount, lane, s_stg[w],
                           pass * 64, pass * 64 + 64);
      continue;
    }
    const int64_t ix = idx - total_g;
    const int2 im = a.item_map[ix / npass];
    const int pass = static_cast<int>(ix % npass);
    const int s = im.x;
    const int n = a.seg_n[s];
    // ids taken above in 64-token tiles
    if (grouped && n >= a.group_min_rows) continue;
    const int nch = ceil_div(n, a.chunk_rows);
    // the forward's items are (token tile, row chunk): take each tile once
    if (im.y % nch != 0) continue;
    const int tile = im.y / nch;
    const int t_begin = a.seg_tok_start[s];
    const int m = a.seg_tok_start[s + 1] - t_begin;
    const int tok0 = t_begin + tile * kTokTile;
    const int mcount = min(kTokTile, m - tile * kTokTile);
    dx_att_mfma<1, 128>(a, a.seg_row_off[s], n, tok0, mcount, lane, s_stg[w],
                        pass * 128, pass * 128 + 128);
  }
}

template <typename T>
__global__ __launch_bounds__(256, 2) void seg_bwd_tile_kernel(BwdArgs a) {
  __shared__ __align__(16) float s_ds[4][16 * kTokTile];
  if (a.header[0] != 0) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n_items = a.header[a.count_slot];
  for (int item = blockIdx.x * 4 + w; item < n_items;
       item += gridDim.x * 4) {
    const int2 im = a.item_map[item];
    const int s = im.x;
    const int nch = ceil_div(a.seg_n[s], a.chunk_rows);
    // the forward's items are (token tile, row chunk): take each tile once
    if (im.y % nch != 0) continue;
    bwd_tile<T>(a, s, im.y / nch, lane, s_ds[w]);
  }
}

// Rows of ids absent from the batch get zero gradients (the column pass
// writes every row of the present ids). Segments are in id order and an
// id's rows are contiguous, so the absent rows are the gaps between
// consecutive segments' row ranges (and before the first, after the last).
// One workgroup lists them in pieces of at most 64 rows (thread t takes a
// run of gaps; a scan of the runs' piece counts places them); then
// zero_rows_kernel clears each piece's dK and dV rows.
__global__ __launch_bounds__(1024) void gap_items_kernel(BwdArgs a) {
  __shared__ int s_part[1024];
  if (a.header[0] != 0) return;
  const int S = a.header[1];
  const int tid = threadIdx.x;
  const int per = (S + 1 + 1023) / 1024;
  const int g0 = tid * per, g1 = min(S + 1, g0 + per);
  auto gap = [&](int g, int64_t& lo, int64_t& hi) {
    lo = g == 0 ? 0 : a.seg_row_off[g - 1] + a.seg_n[g - 1];
    hi = g == S ? a.rows : a.seg_row_off[g];
  };
  int cnt = 0;
  for (int g = g0; g < g1; ++g) {
    int64_t lo, hi;
    gap(g, lo, hi);
    if (hi > lo) cnt += static_cast<int>((hi - lo + 63) / 64);
  }
  s_part[tid] = cnt;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = tid >= o ? s_part[tid - o] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  int off = s_part[tid] - cnt;
  for (int g = g0; g < g1; ++g) {
    int64_t lo, hi;
    gap(g, lo, hi);
    for (int64_t r = lo; r < hi; r += 64)
      a.zero_map[off++] =
          make_int2(static_cast<int>(r), static_cast<int>(min(hi - r, int64_t(64))));
  }
  if (tid == 1023) *a.zero_count = s_part[1023];
}

__global__ __launch_bounds__(256) void zero_rows_kernel(BwdArgs a) {
  if (a.header[0] != 0) return;
  const int n = *a.zero_count;
  const float4 z = {0.f, 0.f, 0.f, 0.f};
  for (int it = blockIdx.x; it < n; it += gridDim.x) {
    const int2 p = a.zero_map[it];
    float4* k = reinterpret_cast<float4*>(a.dK + static_cast<int64_t>(p.x) * a.d);
    float4* v =
        reinterpret_cast<float4*>(a.dV + static_cast<int64_t>(p.x) * a.d_e);
    const int nk = p.y * a.d / 4, nv = p.y * a.d_e / 4;
    for (int i = threadIdx.x; i < nk; i += 256) k[i] = z;
    for (int i = threadIdx.x; i < nv; i += 256) v[i] = z;
  }
}

hipError_t zero_absent_launch(const BwdArgs& a, int64_t items_ub,
                              hipStream_t s) {
  gap_items_kernel<<<1, 1024, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int grid = static_cast<int>(items_ub < 4096 ? items_ub : 4096);
  if (grid > 0) zero_rows_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

// The column pass's work list: every (segment, 64-row block) pair that
// holds rows, in segment order. One workgroup: thread t takes a run of
// consecutive segments, an exclusive scan of the runs' block counts gives
// each run its place, then each thread writes its pairs.
__global__ __launch_bounds__(1024) void rows_items_kernel(BwdArgs a) {
  __shared__ int s_part[1024];
  if (a.header[0] != 0) return;
  const int S = a.header[1];
  const int tid = threadIdx.x;
  const int per = (S + 1023) / 1024;
  const int s0 = tid * per, s1 = min(S, s0 + per);
  int cnt = 0;
  for (int s = s0; s < s1; ++s) cnt += ceil_div(a.seg_n[s], kBwdRowBlk);
  s_part[tid] = cnt;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = tid >= o ? s_part[tid - o] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  int off = s_part[tid] - cnt;
  for (int s = s0; s < s1; ++s) {
    const int nb = ceil_div(a.seg_n[s], kBwdRowBlk);
    for (int jb = 0; jb < nb; ++jb) a.rows_map[off + jb] = make_int2(s, jb);
    off += nb;
  }
  if (tid == 1023) *a.rows_count = s_part[1023];
}

template <typename T>
__global__ __launch_bounds__(256) void seg_bwd_rows_kernel(BwdArgs a) {
  __shared__ __align__(16) float s_ds[kTokTile][kBwdRowBlk];
  __shared__ __align__(16) float s_p[kTokTile][kBwdRowBlk];
  __shared__ int s_tok[kTokTile];
  if (a.header[0] != 0) return;
  const int tid = threadIdx.x;
  const int ncb = ceil_div(a.d + a.d_e, kBwdColBlk);
  const int nitems = *a.rows_count;
  const int64_t total = static_cast<int64_t>(nitems) * ncb;
  const T* X = static_cast<const T*>(a.x);
  for (int64_t idx = blockIdx.x; idx < total; idx += gridDim.x) {
    // index = (item, column block): items are in segment order, which puts
    // the ids with most tokens (the lowest ids of a Zipf-like stream) and
    // their longest blocks on the first workgroups dispatched
    const int2 it = a.rows_map[idx / ncb];
    const int cb = static_cast<int>(idx % ncb);
    const int s = it.x, jb = it.y;
    const int n = a.seg_n[s];
    const int j0 = jb * kBwdRowBlk;
    const int t_begin = a.seg_tok_start[s];
    const int t_end = a.seg_tok_start[s + 1];
    const int64_t r0 = a.seg_row_off[s];
    const int c = cb * kBwdColBlk + tid;
    const bool active = c < a.d + a.d_e;
    const bool isK = c < a.d;
    const int col = isK ? c : c - a.d;
    float acc[kBwdRowBlk];
#pragma unroll
    for (int jj = 0; jj < kBwdRowBlk; ++jj) acc[jj] = 0.f;
    for (int p0 = t_begin; p0 < t_end; p0 += kTokTile) {
      const int cnt = min(kTokTile, t_end - p0);
      __syncthreads();  // the previous batch is consumed
      {
        // 16 tokens x 64 rows of dS and p: one float4 of each per thread
        const int t = tid >> 4, jq = (tid & 15) * 4;
        float4 dv = {0.f, 0.f, 0.f, 0.f}, pv = {0.f, 0.f, 0.f, 0.f};
        if (t < cnt) {
          const int64_t o = static_cast<int64_t>(p0 + t) * a.kst + j0 + jq;
          dv = *reinterpret_cast<const float4*>(a.DSbuf + o);
          pv = *reinterpret_cast<const float4*>(a.Pbuf + o);
        }
        *reinterpret_cast<float4*>(&s_ds[t][jq]) = dv;
        *reinterpret_cast<float4*>(&s_p[t][jq]) = pv;
        if (tid < kTokTile) s_tok[tid] = tid < cnt ? a.perm[p0 + tid] : 0;
      }
      __syncthreads();
      if (active) {
        // this column's value of every token of the batch, all loads issued
        // before the first use
        float vals[kTokTile];
#pragma unroll
        for (int t = 0; t < kTokTile; ++t) {
          vals[t] = 0.f;
          if (t < cnt) {
            const int64_t i = s_tok[t];
            vals[t] = isK ? ld<T>(X, i * a.d + col) : a.dA[i * a.d_e + col];
          }
        }
#pragma unroll
        for (int t = 0; t < kTokTile; ++t) {
          if (t < cnt) {
            const float v = vals[t];
            const float4* w4 = reinterpret_cast<const float4*>(
                isK ? &s_ds[t][0] : &s_p[t][0]);
#pragma unroll
            for (int q = 0; q < kBwdRowBlk / 4; ++q) {
              const float4 wv = w4[q];
              acc[4 * q] = fmaf(wv.x, v, acc[4 * q]);
              acc[4 * q + 1] = fmaf(wv.y, v, acc[4 * q + 1]);
              acc[4 * q + 2] = fmaf(wv.z, v, acc[4 * q + 2]);
              acc[4 * q + 3] = fmaf(wv.w, v, acc[4 * q + 3]);
            }
          }
        }
      }
    }
    if (active) {
      const int jn = min(kBwdRowBlk, n - j0);
#pragma unroll
      for (int jj = 0; jj < kBwdRowBlk; ++jj) {
        if (jj < jn) {
          const int64_t row = r0 + j0 + jj;
          if (isK)
            a.dK[row * a.d + col] = acc[jj];
          else
            a.dV[row * a.d_e + col] = acc[jj];
        }
      }
    }
  }
}

// Column pass on 16x16x32 bf16 MFMA (bf16 x, d a multiple of 256, d_e of
// 64): dK_t = dS^T X_t and dV_t = P^T dA_t as small GEMMs, rows of K_t / V_t
// the M index, columns N, the id's tokens the reduction (blocks of 32). One
// workgroup per (id, 64-row block) pair and 256 columns of [K | V]; wave w
// owns 64 of them (all K or all V) and all 64 rows: 4 x 4 accumulators.
// Per token block the workgroup stages dS (K columns) or p (V columns) of
// its 64 rows transposed in LDS as bf16 hi / lo halves ([row][token], A
// operand: 8 consecutive tokens a lane), each wave stages its 32 token rows
// of x (bf16) or dA (float32, as hi / lo) ([token][column]) and reads the B
// operand with the transposing LDS read. dK = dS_hi x + dS_lo x (x is
// exact in bf16), dV = p_hi dA_hi + p_lo dA_hi + p_hi dA_lo: products of
// bf16 values are exact in float32, the lo halves carry the float32
// operands to about 2^-17. Tokens past the id's last get zero weights.
constexpr int kRAS = 32 + 8;   // A staging row stride (elements)
constexpr int kRBS = 64 + 8;   // B staging row stride (elements)

__global__ __launch_bounds__(256) void seg_bwd_rows_mfma_kernel(BwdArgs a) {
  __shared__ __align__(16) uint16_t s_ahi[64 * kRAS];
  __shared__ __align__(16) uint16_t s_alo[64 * kRAS];
  __shared__ __align__(16) uint16_t s_bhi[4][32 * kRBS];
  __shared__ __align__(16) uint16_t s_blo[4][32 * kRBS];
  if (a.header[0] != 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int trow = 8 * g + (r >> 2), tcol = 4 * (r & 3);
  const int ncb = ceil_div(a.d + a.d_e, kBwdColBlk);
  const int nitems = *a.rows_count;
  const int64_t total = static_cast<int64_t>(nitems) * ncb;
  const uint16_t* X = static_cast<const uint16_t*>(a.x);
  typedef __attribute__((address_space(3))) bwd_v4i16 lds_v4i16;
  for (int64_t idx = blockIdx.x; idx < total; idx += gridDim.x) {
    const int2 it = a.rows_map[idx / ncb];
    const int cb = static_cast<int>(idx % ncb);
    const int s = it.x;
    const int n = a.seg_n[s];
    const int j0 = it.y * kBwdRowBlk;
    const int t_begin = a.seg_tok_start[s];
    const int t_end = a.seg_tok_start[s + 1];
    const int64_t r0 = a.seg_row_off[s];
    // the workgroup's columns are all K (c < d) or all V: 256 divides d
    const bool isK = cb * kBwdColBlk < a.d;
    const int c0 = cb * kBwdColBlk + w * 64;   // this wave's first column
    const bool wave_on = c0 < a.d + a.d_e;
    const int col0 = isK ? c0 : c0 - a.d;      // within K or V
    const float* src_a = isK ? a.DSbuf : a.Pbuf;
    floatx4 acc[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int t0 = t_begin; t0 < t_end; t0 += 32) {
      const int cnt = min(32, t_end - t0);
      __syncthreads();  // the previous block is consumed
      {
        // A: token tt, rows jq .. jq+7 of this block (float32 -> hi / lo),
        // written transposed
        const int tt = tid >> 3, jq = (tid & 7) * 8;
        float v[8];
        if (tt < cnt) {
          const float* p = src_a + static_cast<int64_t>(t0 + tt) * a.kst + j0 + jq;
          const float4 u0 = *reinterpret_cast<const float4*>(p);
          const float4 u1 = *reinterpret_cast<const float4*>(p + 4);
          v[0] = u0.x; v[1] = u0.y; v[2] = u0.z; v[3] = u0.w;
          v[4] = u1.x; v[5] = u1.y; v[6] = u1.z; v[7] = u1.w;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint16_t h = f2bf(v[e]);
          s_ahi[(jq + e) * kRAS + tt] = h;
          s_alo[(jq + e) * kRAS + tt] =
              f2bf(v[e] - __uint_as_float(static_cast<uint32_t>(h) << 16));
        }
      }
      if (wave_on) {
        // B: this wave's 32 token rows x 64 columns
        if (isK) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int ch = q * 64 + lane, tt = ch >> 3, cq = (ch & 7) * 8;
            const int64_t row = a.perm[t0 + min(tt, cnt - 1)];
            const u32x4 u = *reinterpret_cast<const u32x4*>(
                X + row * a.d + col0 + cq);
            *reinterpret_cast<u32x4*>(&s_bhi[w][tt * kRBS + cq]) = u;
          }
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int ch = q * 64 + lane, tt = ch >> 4, cq = (ch & 15) * 4;
            const int64_t row = a.perm[t0 + min(tt, cnt - 1)];
            const float4 u = *reinterpret_cast<const float4*>(
                a.dA + row * a.d_e + col0 + cq);
            const float x[4] = {u.x, u.y, u.z, u.w};
            uint32_t h[2], l[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              h[e] = f2bf2(x[2 * e], x[2 * e + 1]);
              l[e] = f2bf2(x[2 * e] - __uint_as_float(h[e] << 16),
                           x[2 * e + 1] - __uint_as_float(h[e] & 0xffff0000u));
            }
            *reinterpret_cast<uint2*>(&s_bhi[w][tt * kRBS + cq]) =
                make_uint2(h[0], h[1]);
            *reinterpret_cast<uint2*>(&s_blo[w][tt * kRBS + cq]) =
                make_uint2(l[0], l[1]);
          }
        }
      }
      __syncthreads();
      if (wave_on) {
        u32x4 ahi[4], alo[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          ahi[mb] = *reinterpret_cast<const u32x4*>(&s_ahi[(mb * 16 + r) * kRAS + 8 * g]);
          alo[mb] = *reinterpret_cast<const u32x4*>(&s_alo[(mb * 16 + r) * kRAS + 8 * g]);
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const bwd_v4i16 l0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)(&s_bhi[w][trow * kRBS + nb * 16 + tcol]));
          const bwd_v4i16 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)(&s_bhi[w][(trow + 4) * kRBS + nb * 16 + tcol]));
          const uint2 la = __builtin_bit_cast(uint2, l0);
          const uint2 ha = __builtin_bit_cast(uint2, h0);
          const u32x4 bh = u32x4{la.x, la.y, ha.x, ha.y};
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) {
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, ahi[mb]),
                __builtin_bit_cast(bf16x8_t, bh), acc[mb][nb], 0, 0, 0);
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, alo[mb]),
                __builtin_bit_cast(bf16x8_t, bh), acc[mb][nb], 0, 0, 0);
          }
          if (!isK) {
            const bwd_v4i16 l1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4i16*)(&s_blo[w][trow * kRBS + nb * 16 + tcol]));
            const bwd_v4i16 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4i16*)(&s_blo[w][(trow + 4) * kRBS + nb * 16 + tcol]));
            const uint2 lb = __builtin_bit_cast(uint2, l1);
            const uint2 hb = __builtin_bit_cast(uint2, h1);
            const u32x4 bl = u32x4{lb.x, lb.y, hb.x, hb.y};
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8_t, ahi[mb]),
                  __builtin_bit_cast(bf16x8_t, bl), acc[mb][nb], 0, 0, 0);
          }
        }
      }
    }
    if (wave_on) {
      const int jn = min(kBwdRowBlk, n - j0);
      float* dst = isK ? a.dK : a.dV;
      const int64_t ld = isK ? a.d : a.d_e;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int jj = mb * 16 + 4 * g + i;
          if (jj < jn) {
            float* row = dst + (r0 + j0 + jj) * ld + col0 + r;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) row[nb * 16] = acc[mb][nb][i];
          }
        }
    }
  }
}

hipError_t seg_bwd_launch(const BwdArgs& a, int dtype, int items_ub, int S_ub,
                          hipStream_t s) {
  if (items_ub <= 0 || S_ub <= 0) return hipSuccess;
  int grid = ceil_div(items_ub, 4);
  if (grid > 8192) grid = 8192;
  const bool split = dtype == kBF16 && a.d % 128 == 0 && a.chunk_stats;
  if (split) {
    seg_bwd_chunk_kernel<uint16_t, false><<<grid, 256, 0, s>>>(a);
    seg_bwd_chunk_kernel<uint16_t, true><<<grid, 256, 0, s>>>(a);
  } else if (dtype == kBF16) {
    seg_bwd_tile_kernel<uint16_t><<<grid, 256, 0, s>>>(a);
  } else {
    seg_bwd_tile_kernel<float><<<grid, 256, 0, s>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dtype == kBF16 && a.d % 128 == 0) {
    const int64_t g_ub =
        a.group_min_rows > 0 ? group_items_cap(a.B) * 2 * (a.d / 64) : 0;
    const int64_t dx_blocks =
        (static_cast<int64_t>(items_ub) * (a.d / 128) + g_ub + 3) / 4;
    seg_bwd_dx_kernel<<<static_cast<int>(dx_blocks < 8192 ? dx_blocks : 8192),
                        256, 0, s>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  rows_items_kernel<<<1, 1024, 0, s>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t blocks = static_cast<int64_t>(S_ub) *
                         ceil_div(a.d + a.d_e, kBwdColBlk) *
                         ceil_div(a.kst, kBwdRowBlk);
  const int grid2 = static_cast<int>(blocks < 8192 ? blocks : 8192);
  if (dtype == kBF16 && a.d % kBwdColBlk == 0 && a.d_e % 64 == 0)
    seg_bwd_rows_mfma_kernel<<<grid2, 256, 0, s>>>(a);
  else if (dtype == kBF16)
    seg_bwd_rows_kernel<uint16_t><<<grid2, 256, 0, s>>>(a);
  else
    seg_bwd_rows_kernel<float><<<grid2, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace l3
