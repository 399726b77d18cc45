// Group kernel of the segment forward: ids with many rows, large batches.
//
// Same computation as seg_fwd (a_i = V_t^T Softmax(K_t x_i); gist.science
// explainer of "L^3: Large Lookup Layers", Technical Summary, Core
// Architecture, Mathematical Formulation and Context-Dependent Aggregation;
// Systems-Friendly Design, Batch Sorting for the per-id grouping), organised
// for ids whose K_t, V_t slices are large (>= 128 rows of a 2048-wide key):
// one workgroup of eight waves owns an item = (id, tile of up to 64 of its
// tokens) and all of the id's rows (at most 512).
//
//   scores   S = X K_t^T (64 tokens x n rows) on 16x16x32 bf16 MFMA. Wave w
//            owns an even share of the rows (16, 32 or 64 of them); its K
//            fragments stream from global memory straight into registers,
//            a few 32-column steps ahead of the multiply (each K row is used
//            by exactly one wave, so it never touches LDS). The X slice
//            (64 tokens x 128 columns) is shared by
//            all waves, so it is staged in LDS, double buffered, one barrier
//            per slice. Both operands use the same lane -> k assignment.
//   softmax  exact: per-wave row maxima / sums combined through LDS; the
//            weights are written to LDS as bf16 [token][row], rows padded to
//            a multiple of 32 with zeros.
//   values   A (64 tokens x d_e) = P V_t on 16x16x32 bf16 MFMA. Wave w owns
//            columns (d_e/8)w ..; its V block (32 rows x d_e/8 columns per
//            step) is staged row-major in a wave-private LDS buffer and read
//            with the transposing LDS load (ds_read_b64_tr_b16): within a
//            16-lane group, output lane i, slot c receives element i % 4 of
//            source lane 4c + i / 4, so source lanes that read four
//            consecutive columns of rows 8G + s/4 hand every lane eight
//            consecutive rows of one column -- the B operand layout.
//   output   a = A / rowsum, bf16 (and float32 when saving), original order.
// One launch of this kernel runs the whole segment forward of the batch:
// workgroups take items from three device-wide queues (the 128-token items
// of the busiest ids; the 64-token items in id order; the wave items of the
// ids with fewer rows, one per wavefront, run by the same code as the wave
// kernel), half of the workgroups starting with the wave items and half with
// the others, every workgroup then visiting the remaining queues. Every item
// walks the key width from a column slice of its own so that concurrent
// items do not all read the same column offset of their rows (which crowds
// a few memory channels).

#include "l3_device.h"
#include "l3_internal.h"
#include "seg_wave.h"

namespace l3 {

#ifndef L3_WAVE_FIRST_EVERY
#define L3_WAVE_FIRST_EVERY 2
#endif
constexpr int kWaveFirstEvery = L3_WAVE_FIRST_EVERY;
// 64-token items of ids with more rows than this take the busy-id path
constexpr int kGroupAsHotRows = 384;
constexpr int kGW = 8;                 // waves per workgroup
constexpr int kGT = kGroupTok;         // tokens per item
constexpr int kGRows = L3_MAX_ROWS_PER_ID;
constexpr int kSW = 128;               // columns of d per K / X slice
constexpr int kXS = kSW + 8;           // X slice row stride (elements)
constexpr int kPS = kGRows + 8;        // P row stride
constexpr int kVR = 32;                // V rows per value step
constexpr int kCPWMax = 64;            // value columns per wave at most
constexpr int kVS = kCPWMax + 8;       // V staging row stride

typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Maximum / sum of the eight per-wave partials of one token, stored
// contiguously ([token][wave]) so two 16-byte LDS reads fetch them.
__device__ __forceinline__ float max8(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  return fmaxf(fmaxf(fmaxf(a.x, a.y), fmaxf(a.z, a.w)),
               fmaxf(fmaxf(b.x, b.y), fmaxf(b.z, b.w)));
}
__device__ __forceinline__ float sum8(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  return ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
}

__device__ __forceinline__ floatx4 mfma16(const u32x4& a, const u32x4& b,
                                          floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0,
      0, 0);
}

template <int MB, int NBW, int NBV>
__device__ __forceinline__ void group_item(
    const SegGroupArgs& a, int tok0, int mcount, int n, int64_t rowbase,
    int rot,
    uint16_t (*s_x)[kGT * kXS], uint16_t* s_p, uint16_t* s_v,
    float (*red)[kGT][kGW], int* queue, int& next) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int d = a.d;
  const int nsl = d / kSW;

  // ------------------------------------------------------------ scores ---
  // Wave w owns rows 16*NBW*w .. 16*NBW*(w+1)-1, NBW = 1, 2 or 4 blocks of
  // 16 rows chosen from n so that the eight waves share the id's rows
  // evenly. K streams in 32-column steps through a ring of R = 4, 2, 2
  // register slots (NBW = 1, 2, 4): step t's loads are issued R-1 steps
  // before its multiply (the loop is unrolled by R so every slot index is
  // static, and there is no per-wave branch), 1 - 4 KB of K in flight per
  // wave. Deeper rings (up to 16 KB a wave) were slower: they pushed the
  // kernel past 256 registers into spills, and with eight such waves on
  // every CU the memory system is already saturated. Lane group g supplies
  // columns 32t + 8g .. 32t + 8g + 7
  // of its row for both operands. X is staged in 128-column slices in LDS
  // (double buffered, one barrier per slice). A wave past the id's last row
  // re-reads that cached row; its results are masked below.
  constexpr int R = 4 / NBW > 1 ? 4 / NBW : 2;
  const int wrow0 = w * 16 * NBW;
  const bool has_rows = wrow0 < n;
  int koff[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
    koff[nb] = min(wrow0 + nb * 16 + r, n - 1) * d + g * 8;
  const uint16_t* kt = a.K + rowbase * d;
  const int xt = tid >> 3, xc = (tid & 7) * 8;
  const uint16_t* xsrc =
      a.x + static_cast<int64_t>(a.perm[tok0 + min(xt, mcount - 1)]) * d + xc;

  floatx4 acc[MB][NBW];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = d / 32;  // a multiple of 16 (seg_group_ok)
  u32x4 kr[R][NBW];
  // Items walk d from a slice of their own (rot), and within a slice wave w
  // starts at step w % 4: when every wave reads the same column offset of
  // its rows at once, the accesses pile onto a few memory channels (a probe
  // loses a fifth of the bandwidth that way).
  auto rcol = [&](int sl) {
    const int rs = sl + rot;
    return (rs < nsl ? rs : rs - nsl) * kSW;
  };
#define L3_LOAD_K(slot, t)                                               \
  {                                                                      \
    const int tt_ = min((t), nsteps - 1);                                \
    const int col = rcol(tt_ >> 2) + ((tt_ + w) & 3) * 32;               \
    _Pragma("unroll") for (int nb = 0; nb < NBW; ++nb) kr[slot][nb] =    \
        ld16(kt + koff[nb] + col);                                       \
  }
  u32x4 x0 = ld16(xsrc + rcol(0)), x1 = ld16(xsrc + rcol(0) + 64);
  *reinterpret_cast<u32x4*>(&s_x[0][xt * kXS + xc]) = x0;
  *reinterpret_cast<u32x4*>(&s_x[0][xt * kXS + xc + 64]) = x1;
#pragma unroll
  for (int q = 0; q < R - 1; ++q) L3_LOAD_K(q, q)
  {
    const int nx = rcol(min(1, nsl - 1));
    x0 = ld16(xsrc + nx);
    x1 = ld16(xsrc + nx + 64);
  }
  __syncthreads();
  for (int base = 0; base < nsteps; base += R) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int t = base + q;
      L3_LOAD_K((q + R - 1) % R, t + R - 1)
      // keep the loads ahead of this step's multiplies: left alone, the
      // scheduler sinks them past the MFMAs and the ring drains each step
      __builtin_amdgcn_sched_barrier(0);
      // step t is step t % 4 of X slice t / 4 (R need not be a multiple
      // of 4: the slice position comes from t, not from the ring slot)
      const int buf = (t >> 2) & 1;
      u32x4 xf[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        xf[mb] = *reinterpret_cast<const u32x4*>(
            &s_x[buf][(mb * 16 + r) * kXS + ((t + w) & 3) * 32 + g * 8]);
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb][nb] = mfma16(xf[mb], kr[q][nb], acc[mb][nb]);
      if ((t & 3) == 3) {
        // end of X slice t/4: the next slice (in registers) goes to the
        // other buffer, the one after is fetched
        *reinterpret_cast<u32x4*>(&s_x[buf ^ 1][xt * kXS + xc]) = x0;
        *reinterpret_cast<u32x4*>(&s_x[buf ^ 1][xt * kXS + xc + 64]) = x1;
        const int nx = rcol(min((t >> 2) + 2, nsl - 1));
        x0 = ld16(xsrc + nx);
        x1 = ld16(xsrc + nx + 64);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
#undef L3_LOAD_K

  // the workgroup's next item is requested here: the atomic's latency hides
  // behind the rest of this item, and no item waits behind a whole one
  if (tid == 0) next = atomicAdd(queue, 1);

  // ----------------------------------------------------------- softmax ---
  // lane holds S[token mb*16 + 4g + i][row wrow0 + nb*16 + r]
  const int n32 = (n + kVR - 1) / kVR * kVR;
  float mx[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx[mb][i] = -INFINITY;
  if (has_rows) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
      if (wrow0 + nb * 16 + r < n) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            mx[mb][i] = fmaxf(mx[mb][i], acc[mb][nb][i]);
      }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float m = group16_max(mx[mb][i]);
      if (r == 0) red[0][mb * 16 + 4 * g + i][w] = m;
    }
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = mb * 16 + 4 * g + i;
      const float m = max8(&red[0][t][0]);
      mx[mb][i] = m;
    }
  float sm[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm[mb][i] = 0.f;
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int row = wrow0 + nb * 16 + r;
    if (row < n32) {
      const bool valid = row < n;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = valid ? __expf(acc[mb][nb][i] - mx[mb][i]) : 0.f;
          sm[mb][i] += p;
          s_p[(mb * 16 + 4 * g + i) * kPS + row] = f2bf(p);
        }
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s = group16_sum(sm[mb][i]);
      if (r == 0) red[1][mb * 16 + 4 * g + i][w] = s;
    }
  __syncthreads();

  // ------------------------------------------------------------ values ---
  constexpr int CPW = NBV * 16;      // value columns of this wave
  constexpr int CPR = CPW / 8;       // 16-byte chunks per staged row
  constexpr int SPL = (kVR * CPR) / 64;  // staged chunks per lane
  const int col0 = w * CPW;
  const uint16_t* vt = a.V + rowbase * a.d_e + col0;
  const int nst = n32 / kVR;
  u32x4 vreg[SPL];
  int vrow[SPL], vcol[SPL];
#pragma unroll
  for (int q = 0; q < SPL; ++q) {
    const int id = q * 64 + lane;
    vrow[q] = id / CPR;
    vcol[q] = (id % CPR) * 8;
  }
#pragma unroll
  for (int q = 0; q < SPL; ++q)
    vreg[q] = ld16(vt + static_cast<int64_t>(min(vrow[q], n - 1)) * a.d_e +
                   vcol[q]);
#pragma unroll
  for (int q = 0; q < SPL; ++q)
    *reinterpret_cast<u32x4*>(&s_v[vrow[q] * kVS + vcol[q]]) = vreg[q];
#pragma unroll
  for (int q = 0; q < SPL; ++q)
    vreg[q] = ld16(vt + static_cast<int64_t>(min(kVR + vrow[q], n - 1)) *
                            a.d_e + vcol[q]);
  floatx4 acc2[MB][NBV];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBV; ++nb)
      acc2[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
  // transposing-read source position of this lane: rows 8g + r/4 (+4),
  // columns 4 * (r % 4) of each 16-column block
  const int trow = 8 * g + (r >> 2), tcol = 4 * (r & 3);
  for (int st = 0; st < nst; ++st) {
    __builtin_amdgcn_wave_barrier();
    u32x4 pf[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      pf[mb] = *reinterpret_cast<const u32x4*>(
          &s_p[(mb * 16 + r) * kPS + st * kVR + g * 8]);
    u32x4 bf[NBV];
#pragma unroll
    for (int nb = 0; nb < NBV; ++nb) {
      typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16*)(&s_v[trow * kVS + nb * 16 + tcol]));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16*)(&s_v[(trow + 4) * kVS + nb * 16 + tcol]));
      const uint2 l2 = __builtin_bit_cast(uint2, lo);
      const uint2 h2 = __builtin_bit_cast(uint2, hi);
      bf[nb] = u32x4{l2.x, l2.y, h2.x, h2.y};
    }
#pragma unroll
    for (int nb = 0; nb < NBV; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc2[mb][nb] = mfma16(pf[mb], bf[nb], acc2[mb][nb]);
    __builtin_amdgcn_wave_barrier();
    // next step's rows into the (wave-private) staging buffer, then the
    // step after next into registers
#pragma unroll
    for (int q = 0; q < SPL; ++q)
      *reinterpret_cast<u32x4*>(&s_v[vrow[q] * kVS + vcol[q]]) = vreg[q];
    const int nr = min(st + 2, nst - 1) * kVR;
#pragma unroll
    for (int q = 0; q < SPL; ++q)
      vreg[q] = ld16(vt + static_cast<int64_t>(min(nr + vrow[q], n - 1)) *
                              a.d_e + vcol[q]);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ------------------------------------------------------------ output ---
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = mb * 16 + 4 * g + i;
      if (t < mcount) {
        const float l = sum8(&red[1][t][0]);
        const float inv = 1.0f / l;
        const int64_t orig = a.perm[tok0 + t];
#pragma unroll
        for (int nb = 0; nb < NBV; ++nb) {
          const float o = acc2[mb][nb][i] * inv;
          const int64_t idx = orig * a.d_e + col0 + nb * 16 + r;
          __builtin_nontemporal_store(f2bf(o), a.a_out + idx);
          if (a.a_save) a.a_save[idx] = o;
        }
      }
    }
  __syncthreads();
}

// ---------------------------------------------------------------- busy ids ---
// Items of ids with more than kGroupTok tokens hold up to kHotTok tokens, so
// the id's K_t and V_t are read once per 128 tokens. Layout of the shared
// buffer: scores phase {X slice [128][72], K slice [512][72]}, then values
// phase {P [128][520], V staging [8 waves][16][72]} in the same bytes.
//
//   scores  S = X K_t^T as a small GEMM on 32x32x16 bf16 MFMA: wave w owns
//           rows 64w .. 64w+63 of K_t (two 32-row blocks) for all tokens
//           (MB32 blocks of 32). Both operands go through LDS in 64-column
//           slices loaded with whole 128-byte lines per row (8 lanes per
//           row): the MFMA register layout would fetch 16 rows x 64 bytes
//           per load, which halves what the L1 delivers when K_t comes from
//           L2, as it does for the later items of a busy id. The next slice
//           is fetched into registers while the current one is multiplied.
//   softmax exact, as in the 64-token path (per-wave maxima and sums through
//           LDS); weights bf16 in P.
//   values  A = P V_t on 16x16x16 bf16 MFMA, wave w owning d_e/8 columns for
//           all tokens; V_t rows reach the B operand through a wave-private
//           16-row staging buffer and the transposing LDS read, the rows of
//           the next three steps in flight in registers.
constexpr int kHT = kHotTok;           // tokens per busy-id item
constexpr int kHS = 64;                // columns per X / K slice
constexpr int kHL = kHS + 8;           // slice row stride (elements)
constexpr int kHPS = kGRows + 8;       // P row stride
constexpr int kHVR = 16;               // V rows per value step
constexpr int kHRV = 4;                // value steps in flight
constexpr size_t kHotScoreBytes = (size_t)(kHT + kGRows) * kHL * 2;
constexpr size_t kHotValueBytes =
    (size_t)kHT * kHPS * 2 + (size_t)kGW * kHVR * kVS * 2;
constexpr size_t kGroupBytes = (size_t)2 * kGT * kXS * 2 +
                               (size_t)kGT * kPS * 2 +
                               (size_t)kGW * kVR * kVS * 2;
static_assert(kGW * kNBMax * 16 * kTokTile * 2 + kGW * 2 * kTokTile * 4 <=
                  kGT * kXS * 2 * 2,
              "wave item buffers fit in the shared bytes");
constexpr size_t kSmemBytes =
    kHotValueBytes > kGroupBytes ? kHotValueBytes : kGroupBytes;
static_assert(kHotScoreBytes <= kSmemBytes, "scores staging must fit");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t group_rsrc(
    const uint16_t* base, int64_t bytes) {
  // 0x00020000: raw (untyped) 32-bit data format, the usual gfx9 setting
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(base), 0,
      static_cast<int>(bytes > 0x7fffffff ? 0x7fffffff : bytes), 0x00020000);
}

// The thread index through an empty asm: addresses derived from it are
// recomputed per item instead of being hoisted out of the item loop (where
// the hundred-odd lane addresses of the softmax would be spilled).
__device__ __forceinline__ int opaque_int(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <int MB32, int NBV>
__device__ __forceinline__ void hot_item(const SegGroupArgs& a, int tok0,
                                         int mcount, int n, int64_t rowbase,
                                         uint8_t* smem,
                                         float (*red)[kHT][kGW], int rot) {
  const int tid = opaque_int(threadIdx.x), lane = tid & 63, w = tid >> 6;
  const int d = a.d;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  uint16_t* ks = xs + kHT * kHL;

  // ------------------------------------------------------------ scores ---
  // staging: thread -> rows lr + 64q, 16-byte chunk lc of the slice
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  const __amdgpu_buffer_rsrc_t rk =
      group_rsrc(a.K + rowbase * d, static_cast<int64_t>(n) * d * 2);
  int kvo[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) kvo[q] = (min(lr + 64 * q, n - 1) * d + lc) * 2;
  const uint16_t* xp[2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
    xp[q] = a.x +
            static_cast<int64_t>(a.perm[tok0 + min(lr + 64 * q, mcount - 1)]) *
                d + lc;
  u32x4 sx[2], sk[8];
  auto load_slice = [&](int c0) {
#pragma unroll
    for (int q = 0; q < 2; ++q) sx[q] = ld16(xp[q] + c0);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      sk[q] = __builtin_amdgcn_raw_buffer_load_b128(rk, kvo[q], c0 * 2, 0);
  };
  floatx16 acc[MB32][2];
#pragma unroll
  for (int i = 0; i < MB32; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{};
  const int nsl = d / kHS;
  const int r = lane & 31, kh = (lane >> 5) * 8;
  // each item walks d from its own slice (rot), spreading channels
  auto rslice = [&](int sl) {
    const int rs = sl + rot;
    return (rs < nsl ? rs : rs - nsl) * kHS;
  };
  load_slice(rslice(0));
  for (int sl = 0; sl < nsl; ++sl) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q)
      *reinterpret_cast<u32x4*>(&xs[(lr + 64 * q) * kHL + lc]) = sx[q];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      *reinterpret_cast<u32x4*>(&ks[(lr + 64 * q) * kHL + lc]) = sk[q];
    __syncthreads();
    load_slice(rslice(min(sl + 1, nsl - 1)));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < kHS; kk += 16) {
      u32x4 af[MB32], bq[2];
#pragma unroll
      for (int i = 0; i < MB32; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(
            &xs[(32 * i + r) * kHL + kk + kh]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bq[j] = *reinterpret_cast<const u32x4*>(
            &ks[(64 * w + 32 * j + r) * kHL + kk + kh]);
#pragma unroll
      for (int i = 0; i < MB32; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = mfma32_bf16(af[i], bq[j], acc[i][j]);
    }
  }

  // ----------------------------------------------------------- softmax ---
  // acc[i][j][e]: token 32i + 8(e/4) + 4h + e%4, row 64w + 32j + r (h, r:
  // lane half and lane within the half)
  const int h4 = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < MB32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float v = -INFINITY;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (64 * w + 32 * j + r < n) v = fmaxf(v, acc[i][j][e]);
      v = group32_max_hi(v);
      if (r == 31) red[0][32 * i + 8 * (e >> 2) + h4 + (e & 3)][w] = v;
    }
  __syncthreads();
  uint16_t* P = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
  for (int i = 0; i < MB32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int t = 32 * i + 8 * (e >> 2) + h4 + (e & 3);
      const float mxv = max8(&red[0][t][0]);
      float sm = 0.f;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = 64 * w + 32 * j + r;
        const float pv = row < n ? __expf(acc[i][j][e] - mxv) : 0.f;
        sm += pv;
        P[t * kHPS + row] = f2bf(pv);
      }
      sm = group32_sum_hi(sm);
      if (r == 31) red[1][t][w] = sm;
    }
  __syncthreads();

  // ------------------------------------------------------------ values ---
  constexpr int TB = MB32 * 2;          // 16-token blocks
  constexpr int CPW = NBV * 16;         // value columns of this wave
  constexpr int CPR = CPW / 8;          // 16-byte chunks per staged row
  constexpr int NCH = kHVR * CPR;       // chunks per step
  constexpr int SPL = (NCH + 63) / 64;  // chunks per lane
  uint16_t* vs = P + kHT * kHPS + w * (kHVR * kVS);
  const int col0 = w * CPW;
  const uint16_t* vt = a.V + rowbase * a.d_e + col0;
  int vrow[SPL], vcol[SPL];
#pragma unroll
  for (int q = 0; q < SPL; ++q) {
    const int id = min(q * 64 + lane, NCH - 1);
    vrow[q] = id / CPR;
    vcol[q] = (id % CPR) * 8;
  }
  // steps of 16 rows, padded to a multiple of kHRV (P is zero past row n)
  const int nst = ceil_div(ceil_div(n, kHVR), kHRV) * kHRV;
  u32x4 vr[kHRV][SPL];
#define L3_VLOAD(slot, st)                                                  \
  {                                                                         \
    const int slot_ = (slot), row_ = (st) * kHVR;                           \
    _Pragma("unroll") for (int c_ = 0; c_ < SPL; ++c_) vr[slot_][c_] =      \
        ld16(vt + static_cast<int64_t>(min(row_ + vrow[c_], n - 1)) *       \
                      a.d_e + vcol[c_]);                                    \
  }
#pragma unroll
  for (int q = 0; q < kHRV - 1; ++q) L3_VLOAD(q, q)
  floatx4 acc2[TB][NBV];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int cb = 0; cb < NBV; ++cb) acc2[tb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int r16 = lane & 15, g16 = lane >> 4;
  // transposing-read source of this lane: row 4*g16 + r16/4, columns
  // 4 * (r16 % 4) of each 16-column block
  const int trow = 4 * g16 + (r16 >> 2), tcol = 4 * (r16 & 3);
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  for (int base = 0; base < nst; base += kHRV) {
#pragma unroll
    for (int q = 0; q < kHRV; ++q) {
      const int st = base + q;
      L3_VLOAD((q + kHRV - 1) % kHRV, st + kHRV - 1)
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int c = 0; c < SPL; ++c)
        *reinterpret_cast<u32x4*>(&vs[vrow[c] * kVS + vcol[c]]) = vr[q][c];
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_sched_barrier(0);
      v4i16 bq[NBV];
#pragma unroll
      for (int cb = 0; cb < NBV; ++cb)
        bq[cb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(&vs[trow * kVS + cb * 16 + tcol]));
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const v4i16 pa = *reinterpret_cast<const v4i16*>(
            &P[(tb * 16 + r16) * kHPS + st * kHVR + 4 * g16]);
#pragma unroll
        for (int cb = 0; cb < NBV; ++cb)
          acc2[tb][cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
              pa, bq[cb], acc2[tb][cb], 0, 0, 0);
      }
    }
  }
#undef L3_VLOAD

  // ------------------------------------------------------------ output ---
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = tb * 16 + 4 * g16 + i;
      if (t < mcount) {
        const float l = sum8(&red[1][t][0]);
        const float inv = 1.0f / l;
        const int64_t orig = a.perm[tok0 + t];
#pragma unroll
        for (int cb = 0; cb < NBV; ++cb) {
          const float o = acc2[tb][cb][i] * inv;
          const int64_t idx = orig * a.d_e + col0 + cb * 16 + r16;
          __builtin_nontemporal_store(f2bf(o), a.a_out + idx);
          if (a.a_save) a.a_save[idx] = o;
        }
      }
    }
  __syncthreads();
}


// The wave items (ids with fewer rows), one per wavefront from their own
// queue, biggest first, on a workgroup's eight waves (each wave takes its
// next item as soon as its current one is done).
template <int NBV>
__device__ __forceinline__ void wave_pass(const SegGroupArgs& a,
                                          uint8_t* smem, int* work) {
  typedef Types<true, false>::P PT;
  constexpr int kEPL = NBV == 1 ? 2 : 4;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  PT* P = reinterpret_cast<PT*>(smem) + wv * (kNBMax * 16 * kTokTile);
  float* ml = reinterpret_cast<float*>(
                  smem + kGW * kNBMax * 16 * kTokTile * sizeof(PT)) +
              wv * 2 * kTokTile;
  const int n_wave = a.wave.header[a.wave.count_slot];
  int wi = 0;
  if (lane == 0) wi = atomicAdd(&work[5], 1);
  wi = __shfl(wi, 0);
  while (wi < n_wave)
    wi = wave_item<true, kEPL, false>(a.wave, wi, lane, P, ml, &work[5]);
}

template <int NBV>
__global__ __launch_bounds__(512, 1) void seg_group_kernel(SegGroupArgs a) {
  __shared__ __align__(16) uint8_t smem[kSmemBytes];
  __shared__ __align__(16) float s_red[2][kHT][kGW];
  if (a.header[0] != 0) return;
  // 64-token path: X slices, P and V staging carved from the same bytes
  uint16_t (*s_x)[kGT * kXS] = reinterpret_cast<uint16_t (*)[kGT * kXS]>(smem);
  uint16_t* s_p = reinterpret_cast<uint16_t*>(smem) + 2 * kGT * kXS;
  uint16_t* s_v = s_p + kGT * kPS;
  float (*red64)[kGT][kGW] = reinterpret_cast<float (*)[kGT][kGW]>(&s_red[0][0][0]);
  const int n_items = a.header[3];
  uint16_t* my_v = s_v + (threadIdx.x >> 6) * (kVR * kVS);
  // Passes over device-wide work queues: the 128-token items of ids with
  // more than kGroupTok tokens (one list per XCD), the 64-token items, the wave
  // items (separate loops keep the paths' registers apart). A workgroup
  // requests its next 128-token item when it starts one, its next 64-token
  // or wave item once the current item's scores are done, and reads the
  // answer when the item ends, so the atomic's latency overlaps the work;
  // the last workgroup out resets the queues for the next launch.
  __shared__ int s_next;
  int* work = a.work;
  // this XCD's list of 128-token items and its queue
  const int xl = blockIdx.x % kXcds;
  const int n_hot = a.header[16 + xl];
  int* hot_queue = &work[20 + xl];
  const int2* hot_list = a.hitem_map + static_cast<int64_t>(xl) * a.hcap;
  // Half of the workgroups (alternate groups of eight: every XCD gets its
  // share) start with the wave items, the rest with the busy ids' and the
  // 64-token items; every workgroup then visits the other queues. The wave
  // items' latency-bound tail (ids with a few rows) so runs beside the
  // streaming 64-token items instead of after them.
  const bool wave_first = a.wave.header && ((blockIdx.x >> 3) % kWaveFirstEvery) == 0;
  if (wave_first) {
    wave_pass<NBV>(a, smem, work);
    __syncthreads();
  }
  if (threadIdx.x == 0) s_next = atomicAdd(hot_queue, 1);
  __syncthreads();
  for (int hi = s_next; hi < n_hot;) {
    __syncthreads();  // every wave has read s_next
    int next = 0;
    if (threadIdx.x == 0) next = atomicAdd(hot_queue, 1);
    const int2 im = hot_list[hi];
    const int s = im.x, tile = im.y;
    const int t_begin = a.seg_tok_start[s];
    const int m = a.seg_tok_start[s + 1] - t_begin;
    const int n = a.seg_n[s];
    const int64_t rowbase = a.seg_row_off[s];
    const int tok0 = t_begin + tile * kHT;
    const int mcount = min(kHT, m - tile * kHT);
    const int rot = (s * 7 + tile * 3) % (a.d / kHS);
    if (mcount > 64)
      hot_item<4, NBV>(a, tok0, mcount, n, rowbase, smem, s_red, rot);
    else
      hot_item<2, NBV>(a, tok0, mcount, n, rowbase, smem, s_red, rot);
    if (threadIdx.x == 0) s_next = next;
    __syncthreads();
    hi = s_next;
  }
  __syncthreads();
  // 64-token items in id order (the ids with most rows first); the
  // 128-token items met on the way are skipped
  if (threadIdx.x == 0) s_next = atomicAdd(&work[0], 1);
  __syncthreads();
  int item = s_next;
  while (item < n_items) {
    __syncthreads();  // every wave has read s_next
    int next = 0;
    const int2 im = a.gitem_map[item];
    const int s = im.x;
    const int t_begin = a.seg_tok_start[s];
    const int m = a.seg_tok_start[s + 1] - t_begin;
    if (m <= kGT && a.seg_n[s] > kGroupAsHotRows) {
      // ids with most of the 512 rows take the busy-id path: whole-line K
      // loads staged through LDS stream faster (≈ 22 against ≈ 19 GB/s a
      // CU), and with > 384 rows its 64-row-per-wave split keeps the eight
      // waves busy
      if (threadIdx.x == 0) next = atomicAdd(&work[0], 1);
      hot_item<2, NBV>(a, t_begin, m, a.seg_n[s], a.seg_row_off[s], smem,
                       s_red, (s * 7) % (a.d / kHS));
    } else if (m <= kGT) {
    const int n = a.seg_n[s];
    const int64_t rowbase = a.seg_row_off[s];
    const int tok0 = t_begin;
    const int mcount = m;
    const int rot = (s * 7) % (a.d / kSW);
#define L3_ITEM(MB, NBW) \
  group_item<MB, NBW, NBV>(a, tok0, mcount, n, rowbase, rot, s_x, s_p, my_v, \
                           red64, &work[0], next)
#define L3_ROWS(MB)        \
  if (n <= 128)            \
    L3_ITEM(MB, 1);        \
  else if (n <= 256)       \
    L3_ITEM(MB, 2);        \
  else                     \
    L3_ITEM(MB, 4);
    if (mcount <= 16) {
      L3_ROWS(1)
    } else if (mcount <= 32) {
      L3_ROWS(2)
    } else {
      L3_ROWS(4)
    }
#undef L3_ROWS
#undef L3_ITEM
    } else if (threadIdx.x == 0) {
      next = atomicAdd(&work[0], 1);
    }
    if (threadIdx.x == 0) s_next = next;
    __syncthreads();
    item = s_next;
  }
  __syncthreads();
  if (a.wave.header && !wave_first) {
    wave_pass<NBV>(a, smem, work);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int left = atomicAdd(&work[1], 1);
    if (left == static_cast<int>(gridDim.x) - 1) {
      atomicExch(&work[0], 0);
      atomicExch(&work[1], 0);
      atomicExch(&work[5], 0);
      for (int x = 0; x < kXcds; ++x) atomicExch(&work[20 + x], 0);
    }
  }
}

bool seg_group_ok(int d, int d_e) {
  // d: whole 16-step K rings (32 columns a step); d_e: one, two or four
  // 16-column value blocks per wave
  return d % 512 == 0 && (d_e == 128 || d_e == 256 || d_e == 512);
}

hipError_t seg_group_launch(const SegGroupArgs& a, int items_ub,
                            hipStream_t s) {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                              dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  int grid = items_ub < cus ? items_ub : cus;
  if (grid > 8) grid &= ~7;
  if (grid < 1) return hipSuccess;
  switch (a.d_e / 128) {
    case 1:
      seg_group_kernel<1><<<grid, 512, 0, s>>>(a);
      break;
    case 2:
      seg_group_kernel<2><<<grid, 512, 0, s>>>(a);
      break;
    default:
      seg_group_kernel<4><<<grid, 512, 0, s>>>(a);
      break;
  }
  return hipGetLastError();
}

}  // namespace l3
