// Wave work items of the segment forward (a_i = V_t^T Softmax(K_t x_i) for
// up to 16 tokens of one id and up to 128 of its rows on one wavefront),
// shared by the wave kernel and the group kernel's wave-item pass.
//
//   1. scores S = X K_chunk^T on 16x16 MFMA blocks, operands streamed from
//      global memory into registers. bf16: 32-column steps (lane group g
//      holds columns 8g .. 8g+7 of row l & 15, the MFMA's own k layout)
//      through a ring of 8 / 4 / 2 steps for chunks of <= 16 / <= 32 / more
//      rows. f32: 16-column steps of the 16x16x4 MFMA (lane group g holds
//      columns 4g .. 4g+3; four MFMAs, one per element, the same lane -> k
//      assignment for both operands). A single token with d = 512, 1024 or
//      2048 takes whole-row loads instead (scores_softmax_1tok);
//   2. exact softmax over the chunk (row max and row sum across the 16
//      lanes holding a row), unnormalised weights to this wave's LDS (fp16
//      for bf16 inputs, f32 for f32 inputs and the saving forward), laid
//      out [row j][token];
//   3. aggregation acc[t][e] += p[t][j] * V[j][e] on the vector ALU: lane l
//      owns columns e = l*EPL .. l*EPL+EPL-1 of a 64*EPL-column pass, V
//      rows in two 8-row half bursts, the token loop bounded by the tile;
//   4. single chunk: a = acc / rowsum, written in original token order
//      (bf16 rows with streaming stores); several chunks: (max, sum, acc)
//      partials for the combine kernel.
//
// gist.science explainer of "L^3: Large Lookup Layers", Technical Summary,
// Core Architecture, Mathematical Formulation (the attention of x over
// K_t, V_t) and Systems-Friendly Design, Batch Sorting (tokens grouped by id
// share one read of the id's rows).
#pragma once

#include <type_traits>

#include "l3_device.h"
#include "l3_internal.h"

namespace l3 {

constexpr int kNBMax = kWaveMaxRows / 16;  // 16-row blocks per item
constexpr int kVHalf = 8;                  // V rows per half burst

// Storage of the inputs (T) and of the unnormalised weights in LDS (P):
// fp16 weights for bf16 inputs, float32 for float32 inputs and whenever the
// float32 aggregate is saved for the backward pass (P32).
template <bool BF16, bool P32 = false>
struct Types;
template <bool P32>
struct Types<true, P32> {
  typedef uint16_t T;
  typedef typename std::conditional<P32, float, _Float16>::type P;
};
template <bool P32>
struct Types<false, P32> {
  typedef float T;
  typedef float P;
};

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// ---- scores --------------------------------------------------------------
template <int NB, int R>
__device__ __forceinline__ void scores_bf16(const uint16_t* __restrict__ xr,
                                            const uint16_t* __restrict__ kt,
                                            int d, int nc, int r, int g,
                                            int rot,
                                            floatx4 (&acc)[kNBMax]) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
  int koff[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    koff[nb] = min(nb * 16 + r, nc - 1) * d + g * 8;
  const uint16_t* xp = xr + g * 8;
  const int nsteps = d / 32;  // a multiple of R
  // ring of R register slots: step t's loads are issued R-1 steps ahead of
  // its multiply; the loop is unrolled by R so slot indices are static
  u32x4 xs[R], ks[R][NB];
  // the item walks d from step rot (items reading the same column offset
  // of their rows at once crowd a few memory channels)
#define L3_LOAD(slot, t)                                              \
  {                                                                   \
    const int t_ = min((t), nsteps - 1) + rot;                        \
    const int c = (t_ < nsteps ? t_ : t_ - nsteps) * 32;              \
    xs[slot] = ld16(xp + c);                                          \
    _Pragma("unroll") for (int nb = 0; nb < NB; ++nb) ks[slot][nb] =  \
        ld16(kt + koff[nb] + c);                                      \
  }
#pragma unroll
  for (int q = 0; q < R - 1; ++q) L3_LOAD(q, q)
  for (int base = 0; base < nsteps; base += R) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      L3_LOAD((q + R - 1) % R, base + q + R - 1)
      // keep the loads ahead of this step's multiplies: left alone, the
      // scheduler sinks them past the MFMAs and the ring drains each step
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, xs[q]),
            __builtin_bit_cast(bf16x8_t, ks[q][nb]), acc[nb], 0, 0, 0);
    }
  }
#undef L3_LOAD
}

template <int NB>
__device__ __forceinline__ void scores_f32(const float* __restrict__ xr,
                                           const float* __restrict__ kt,
                                           int d, int nc, int r, int g,
                                           floatx4 (&acc)[kNBMax]) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
  int koff[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    koff[nb] = min(nb * 16 + r, nc - 1) * d + g * 4;
  const float* xp = xr + g * 4;
  for (int kc = 0; kc < d; kc += 16) {
    const float4 xv = *reinterpret_cast<const float4*>(xp + kc);
    float4 kv[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      kv[nb] = *reinterpret_cast<const float4*>(kt + koff[nb] + kc);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      acc[nb] = mfma_f32(xv.x, kv[nb].x, acc[nb]);
      acc[nb] = mfma_f32(xv.y, kv[nb].y, acc[nb]);
      acc[nb] = mfma_f32(xv.z, kv[nb].z, acc[nb]);
      acc[nb] = mfma_f32(xv.w, kv[nb].w, acc[nb]);
    }
  }
}

// ---- softmax --------------------------------------------------------------
// Row 4g+i of the tile is token 4g+i; column nb*16 + r is row j of the chunk.
template <int NB, typename PT>
__device__ __forceinline__ void softmax_rows(floatx4 (&acc)[kNBMax], int nc,
                                             int r, int g, PT* P, float* ml) {
  float mx[4], sm[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mx[i] = -INFINITY;
    sm[i] = 0.f;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if (nb * 16 + r < nc) {
#pragma unroll
      for (int i = 0; i < 4; ++i) mx[i] = fmaxf(mx[i], acc[nb][i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) mx[i] = group16_max(mx[i]);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int col = nb * 16 + r;
    if (col < nc) {
      PT* dst = P + col * kTokTile + 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __expf(acc[nb][i] - mx[i]);
        sm[i] += p;
        dst[i] = static_cast<PT>(p);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) sm[i] = group16_sum(sm[i]);
  if (r == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ml[(4 * g + i) * 2] = mx[i];
      ml[(4 * g + i) * 2 + 1] = sm[i];
    }
  }
}

template <int NB, bool BF16, typename PT>
__device__ __forceinline__ void scores_softmax(
    const typename Types<BF16>::T* xr, const typename Types<BF16>::T* kt,
    int d, int nc, int r, int g, int rot, PT* P, float* ml) {
  floatx4 acc[kNBMax];
  if constexpr (BF16) {
    // deeper rings where few rows leave registers free
    constexpr int R = NB == 1 ? 8 : (NB == 2 ? 4 : 2);
    if (R > 2 && (d / 32) % R == 0)
      scores_bf16<NB, R>(xr, kt, d, nc, r, g, rot, acc);
    else
      scores_bf16<NB, 2>(xr, kt, d, nc, r, g, rot, acc);
  } else
    scores_f32<NB>(xr, kt, d, nc, r, g, acc);
  softmax_rows<NB>(acc, nc, r, g, P, ml);
}

// Scores and softmax of an item with a single token (bf16, d = 512 DC): the
// token's x row and each K row are read whole, lane l holding columns
// 512q + 8l .. 512q + 8l + 7 (every load instruction covers 1 KB of one
// row), K rows in batches of RB with NR batches in flight; each score is a
// wave-wide sum. The MFMA layout would spend 15 of its 16 token lanes on
// copies of the one token and walk d in 32-column steps; here a whole row
// arrives per batch. Raw scores are parked in this wave's P buffer as
// float, then replaced by the unnormalised weights (same layout and
// precision as softmax_rows: token 0 of each row).
template <int DC, typename PT>
__device__ __forceinline__ void scores_softmax_1tok(
    const uint16_t* __restrict__ xr, const uint16_t* __restrict__ kt, int d,
    int nc, int lane, PT* P, float* ml) {
  constexpr int RB = 2, NR = 4;
  float xf[DC][8];
#pragma unroll
  for (int q = 0; q < DC; ++q) {
    const u32x4 v = ld16(xr + q * 512 + lane * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xf[q][2 * e] = __uint_as_float(v[e] << 16);
      xf[q][2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
    }
  }
  const int nb = ceil_div(nc, RB);
  u32x4 kb[NR][RB][DC];
#define L3_KLOAD(slot, b)                                                  \
  if ((b) < nb) {                                                          \
    _Pragma("unroll") for (int r_ = 0; r_ < RB; ++r_) {                    \
      const int64_t row_ = min((b) * RB + r_, nc - 1);                     \
      _Pragma("unroll") for (int q_ = 0; q_ < DC; ++q_) kb[slot][r_][q_] = \
          ld16(kt + row_ * d + q_ * 512 + lane * 8);                       \
    }                                                                      \
  }
#pragma unroll
  for (int q = 0; q < NR - 1; ++q) L3_KLOAD(q, q)
  float* S = reinterpret_cast<float*>(P);
  float mx = -INFINITY;
  for (int base = 0; base < nb; base += NR) {
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      const int b = base + q;
      L3_KLOAD((q + NR - 1) % NR, b + NR - 1)
      __builtin_amdgcn_sched_barrier(0);
      if (b < nb) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          float dot = 0.f;
#pragma unroll
          for (int c = 0; c < DC; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t u = kb[q][r][c][e];
              dot = fmaf(xf[c][2 * e], __uint_as_float(u << 16), dot);
              dot = fmaf(xf[c][2 * e + 1], __uint_as_float(u & 0xffff0000u),
                         dot);
            }
          const float sc = wave_sum(dot);
          const int j = b * RB + r;
          if (j < nc) {
            mx = fmaxf(mx, sc);
            if (lane == 0) S[j] = sc;
          }
        }
      }
    }
  }
#undef L3_KLOAD
  __builtin_amdgcn_wave_barrier();
  // nc <= 128: lane l owns rows l and l + 64
  const float s0 = lane < nc ? S[lane] : -INFINITY;
  const float s1 = lane + 64 < nc ? S[lane + 64] : -INFINITY;
  const float p0 = lane < nc ? __expf(s0 - mx) : 0.f;
  const float p1 = lane + 64 < nc ? __expf(s1 - mx) : 0.f;
  const float sm = wave_sum(p0 + p1);
  __builtin_amdgcn_wave_barrier();
  if (lane < nc) P[lane * kTokTile] = static_cast<PT>(p0);
  if (lane + 64 < nc) P[(lane + 64) * kTokTile] = static_cast<PT>(p1);
  if (lane == 0) {
    ml[0] = mx;
    ml[1] = sm;
  }
}

// ---- aggregation ------------------------------------------------------------
// EPL values of one row for this lane, as raw storage words.
template <int EPL, bool BF16>
struct RowWords {
  static constexpr int kWords = BF16 ? (EPL + 1) / 2 : EPL;
  uint32_t w[kWords];
};

template <int EPL, bool BF16>
__device__ __forceinline__ void load_words(
    const typename Types<BF16>::T* p, RowWords<EPL, BF16>& v) {
  if constexpr (BF16) {
    if constexpr (EPL == 8) {
      const u32x4 u = ld16(p);
#pragma unroll
      for (int e = 0; e < 4; ++e) v.w[e] = u[e];
    } else if constexpr (EPL == 4) {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      v.w[0] = u.x;
      v.w[1] = u.y;
    } else if constexpr (EPL == 2) {
      v.w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
      v.w[0] = *reinterpret_cast<const uint16_t*>(p);
    }
  } else {
    if constexpr (EPL == 4) {
      const u32x4 u = ld16(p);
#pragma unroll
      for (int e = 0; e < 4; ++e) v.w[e] = u[e];
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        v.w[e] = __float_as_uint(reinterpret_cast<const float*>(p)[e]);
    }
  }
}

template <int EPL, bool BF16>
__device__ __forceinline__ float word_value(const RowWords<EPL, BF16>& v,
                                            int e) {
  if constexpr (BF16) {
    if constexpr (EPL == 1) return __uint_as_float(v.w[0] << 16);
    const uint32_t u = v.w[e >> 1];
    return __uint_as_float((e & 1) ? (u & 0xffff0000u) : (u << 16));
  } else {
    return __uint_as_float(v.w[e]);
  }
}

template <int EPL, typename T>
__device__ __forceinline__ void store_row(T* dst, const float (&v)[EPL]);
// bf16 rows of a are written with streaming (non-temporal) stores: the W_up
// GEMM reads them once, much later.
template <int EPL>
__device__ __forceinline__ void store_row(uint16_t* dst,
                                          const float (&v)[EPL]) {
  if constexpr (EPL == 8) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = f2bf2(v[2 * e], v[2 * e + 1]);
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(dst));
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      __builtin_nontemporal_store(f2bf(v[e]), dst + e);
  }
}
template <int EPL>
__device__ __forceinline__ void store_row(float* dst, const float (&v)[EPL]) {
#pragma unroll
  for (int e = 0; e < EPL; ++e) dst[e] = v[e];
}

template <int MTOK, int EPL, bool BF16, typename PT>
__device__ __forceinline__ void aggregate_and_store(
    const SegFwdArgs& a, const typename Types<BF16>::T* vt, int nc,
    const PT* P, const float* ml, int tok0, int mcount,
    int nch, int chunk, int lane) {
  typedef typename Types<BF16>::T T;
  const int passes = a.d_e / (64 * EPL);
  for (int ps = 0; ps < passes; ++ps) {
    const int e0 = ps * 64 * EPL + lane * EPL;
    const T* vp = vt + e0;
    float acc[MTOK][EPL];
#pragma unroll
    for (int t = 0; t < MTOK; ++t)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[t][e] = 0.f;
    // V rows in two half bursts: the next half is in flight while the
    // current one is used (rows past the chunk repeat its last row; their
    // weights are never read)
    RowWords<EPL, BF16> va[kVHalf], vb[kVHalf];
#define L3_VLOAD(dst, j)                                                  \
  _Pragma("unroll") for (int q = 0; q < kVHalf; ++q) load_words<EPL, BF16>( \
      vp + static_cast<int64_t>(min((j) + q, nc - 1)) * a.d_e, dst[q]);
#define L3_VUSE(src, j)                                                   \
  {                                                                       \
    const int jn = min(kVHalf, nc - (j));                                 \
    _Pragma("unroll") for (int q = 0; q < kVHalf; ++q) {                  \
      if (q < jn) {                                                       \
        const PT* pj = P + ((j) + q) * kTokTile;                          \
        _Pragma("unroll") for (int t = 0; t < MTOK; ++t) {                \
          const float p = static_cast<float>(pj[t]);                      \
          _Pragma("unroll") for (int e = 0; e < EPL; ++e) acc[t][e] =     \
              fmaf(p, word_value<EPL, BF16>(src[q], e), acc[t][e]);       \
        }                                                                 \
      }                                                                   \
    }                                                                     \
  }
    L3_VLOAD(va, 0)
    for (int j0 = 0; j0 < nc; j0 += 2 * kVHalf) {
      L3_VLOAD(vb, j0 + kVHalf)
      __builtin_amdgcn_sched_barrier(0);
      L3_VUSE(va, j0)
      __builtin_amdgcn_sched_barrier(0);
      L3_VLOAD(va, j0 + 2 * kVHalf)
      __builtin_amdgcn_sched_barrier(0);
      L3_VUSE(vb, j0 + kVHalf)
      __builtin_amdgcn_sched_barrier(0);
    }
#undef L3_VLOAD
#undef L3_VUSE
#pragma unroll
    for (int t = 0; t < MTOK; ++t) {
      if (t < mcount) {
        const int pos = tok0 + t;
        if (nch == 1) {
          const float inv = 1.0f / ml[2 * t + 1];
          float o[EPL];
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[e] = acc[t][e] * inv;
          const int64_t orig = a.perm[pos];
          store_row<EPL>(static_cast<T*>(a.a_out) + orig * a.d_e + e0, o);
          if (a.a_save) store_row<EPL>(a.a_save + orig * a.d_e + e0, o);
        } else {
          const int64_t slot =
              static_cast<int64_t>(pos) * a.nch_max + chunk;
          store_row<EPL>(a.part + slot * a.d_e + e0, acc[t]);
          if (ps == 0 && lane == 0) {
            a.part_ml[slot * 2] = ml[2 * t];
            a.part_ml[slot * 2 + 1] = ml[2 * t + 1];
          }
        }
      }
    }
  }
}

// One work item (segment, tile of <= 16 tokens, chunk of <= 128 rows) on
// one wavefront: scores, softmax, aggregation, output. P and ml are this
// wave's LDS buffers. With a queue, the wave's next item is requested once
// the scores are done (the atomic's latency hides behind the aggregation,
// and no item waits behind a long one) and returned; else returns 0.
template <bool BF16, int EPL, bool P32>
__device__ __forceinline__ int wave_item(
    const SegFwdArgs& a, int item, int lane,
    typename Types<BF16, P32>::P* P, float* ml, int* queue = nullptr) {
  typedef typename Types<BF16>::T T;
  typedef typename Types<BF16, P32>::P PT;
  const int r = lane & 15, g = lane >> 4;
  const T* X = static_cast<const T*>(a.x);
  const T* K = static_cast<const T*>(a.K);
  const T* V = static_cast<const T*>(a.V);
  const int2 im = a.item_map[item];
  const int s = im.x, local = im.y;
  const int t_begin = a.seg_tok_start[s];
  const int m = a.seg_tok_start[s + 1] - t_begin;
  const int n = a.seg_n[s];
  const int nch = ceil_div(n, a.chunk_rows);
  const int tile = local / nch, chunk = local - tile * nch;
  const int tok0 = t_begin + tile * kTokTile;
  const int mcount = min(kTokTile, m - tile * kTokTile);
  const int j0 = chunk * a.chunk_rows;
  const int nc = min(a.chunk_rows, n - j0);
  const int64_t rowbase = a.seg_row_off[s] + j0;

  const int64_t xrow = a.perm[tok0 + min(r, mcount - 1)];
  const T* xr = X + xrow * a.d;
  const T* kt = K + rowbase * a.d;
  const int nbc = ceil_div(nc, 16);
  const int rot = (s * 13 + local * 5) % (a.d / 32);
  __builtin_amdgcn_wave_barrier();
  if constexpr (BF16) {
    // a single token with whole-row loads (d = 512, 1024 or 2048)
    const int dc = a.d >> 9;
    if (mcount == 1 && (a.d & 511) == 0 && dc <= 4 && dc != 3) {
      if (dc == 4)
        scores_softmax_1tok<4, PT>(xr, kt, a.d, nc, lane, P, ml);
      else if (dc == 2)
        scores_softmax_1tok<2, PT>(xr, kt, a.d, nc, lane, P, ml);
      else
        scores_softmax_1tok<1, PT>(xr, kt, a.d, nc, lane, P, ml);
      __builtin_amdgcn_wave_barrier();
      int next = 0;
      if (queue && lane == 0) next = atomicAdd(queue, 1);
      const T* vt = V + rowbase * a.d_e;
      // eight value columns per lane when d_e is a multiple of 512
      if (EPL == 4 && (a.d_e & 511) == 0)
        aggregate_and_store<1, 8, BF16, PT>(a, vt, nc, P, ml, tok0, 1, nch,
                                            chunk, lane);
      else
        aggregate_and_store<1, EPL, BF16, PT>(a, vt, nc, P, ml, tok0, 1, nch,
                                              chunk, lane);
      return __shfl(next, 0);
    }
  }
  if (nbc <= 1)
    scores_softmax<1, BF16, PT>(xr, kt, a.d, nc, r, g, rot, P, ml);
  else if (nbc <= 2)
    scores_softmax<2, BF16, PT>(xr, kt, a.d, nc, r, g, rot, P, ml);
  else if (nbc <= 4)
    scores_softmax<4, BF16, PT>(xr, kt, a.d, nc, r, g, rot, P, ml);
  else
    scores_softmax<8, BF16, PT>(xr, kt, a.d, nc, r, g, rot, P, ml);
  __builtin_amdgcn_wave_barrier();
  int next = 0;
  if (queue && lane == 0) next = atomicAdd(queue, 1);

  const T* vt = V + rowbase * a.d_e;
#define L3_AGG(N)                                                        \
  aggregate_and_store<N, EPL, BF16, PT>(a, vt, nc, P, ml, tok0, mcount,  \
                                        nch, chunk, lane)
  if (mcount <= 1)
    L3_AGG(1);
  else if (mcount <= 2)
    L3_AGG(2);
  else if (mcount <= 4)
    L3_AGG(4);
  else if (mcount <= 8)
    L3_AGG(8);
  else
    L3_AGG(16);
#undef L3_AGG
  return __shfl(next, 0);
}

}  // namespace l3
