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
//            up to fifteen 32-column steps ahead of the multiply (each K row
//            is used by exactly one wave, so it never touches LDS). The X slice (64 tokens x 128 columns) is shared by
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
// Items are walked in an XCD-major order so the tiles of one id run on
// workgroups of one XCD and share its L2.

#include "l3_device.h"
#include "l3_internal.h"

namespace l3 {

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

__device__ __forceinline__ floatx4 mfma16(const u32x4& a, const u32x4& b,
                                          floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0,
      0, 0);
}

template <int MB, int NBW, int NBV>
__device__ __forceinline__ void group_item(
    const SegGroupArgs& a, int tok0, int mcount, int n, int64_t rowbase,
    uint16_t (*s_x)[kGT * kXS], uint16_t* s_p, uint16_t* s_v,
    float (*red)[kGW][kGT]) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int d = a.d;
  const int nsl = d / kSW;

  // ------------------------------------------------------------ scores ---
  // Wave w owns rows 16*NBW*w .. 16*NBW*(w+1)-1, NBW = 1, 2 or 4 blocks of
  // 16 rows chosen from n so that the eight waves share the id's rows
  // evenly. K streams in 32-column steps through a ring of R = 16 / NBW
  // register slots: step t's loads are issued R-1 steps before its multiply
  // (the loop is unrolled by R so every slot index is static, and there is
  // no per-wave branch), which keeps 15 .. 12 KB of K in flight per wave
  // whatever NBW is. Lane group g supplies columns 32t + 8g .. 32t + 8g + 7
  // of its row for both operands. X is staged in 128-column slices in LDS
  // (double buffered, one barrier per slice). A wave past the id's last row
  // re-reads that cached row; its results are masked below.
  constexpr int R = 16 / NBW;
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
#define L3_LOAD_K(slot, t)                                               \
  {                                                                      \
    const int col = min((t), nsteps - 1) * 32;                           \
    _Pragma("unroll") for (int nb = 0; nb < NBW; ++nb) kr[slot][nb] =    \
        ld16(kt + koff[nb] + col);                                       \
  }
  u32x4 x0 = ld16(xsrc), x1 = ld16(xsrc + 64);
  *reinterpret_cast<u32x4*>(&s_x[0][xt * kXS + xc]) = x0;
  *reinterpret_cast<u32x4*>(&s_x[0][xt * kXS + xc + 64]) = x1;
#pragma unroll
  for (int q = 0; q < R - 1; ++q) L3_LOAD_K(q, q)
  {
    const int nx = min(1, nsl - 1) * kSW;
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
      const int buf = (t >> 2) & 1;
      u32x4 xf[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        xf[mb] = *reinterpret_cast<const u32x4*>(
            &s_x[buf][(mb * 16 + r) * kXS + (q & 3) * 32 + g * 8]);
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb][nb] = mfma16(xf[mb], kr[q][nb], acc[mb][nb]);
      if ((q & 3) == 3) {
        // end of X slice t/4: the next slice (in registers) goes to the
        // other buffer, the one after is fetched
        *reinterpret_cast<u32x4*>(&s_x[buf ^ 1][xt * kXS + xc]) = x0;
        *reinterpret_cast<u32x4*>(&s_x[buf ^ 1][xt * kXS + xc + 64]) = x1;
        const int nx = min((t >> 2) + 2, nsl - 1) * kSW;
        x0 = ld16(xsrc + nx);
        x1 = ld16(xsrc + nx + 64);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
#undef L3_LOAD_K

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
      if (r == 0) red[0][w][mb * 16 + 4 * g + i] = m;
    }
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = mb * 16 + 4 * g + i;
      float m = red[0][0][t];
#pragma unroll
      for (int v = 1; v < kGW; ++v) m = fmaxf(m, red[0][v][t]);
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
      if (r == 0) red[1][w][mb * 16 + 4 * g + i] = s;
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
        float l = 0.f;
#pragma unroll
        for (int v = 0; v < kGW; ++v) l += red[1][v][t];
        const float inv = 1.0f / l;
        const int64_t orig = a.perm[tok0 + t];
#pragma unroll
        for (int nb = 0; nb < NBV; ++nb) {
          const float o = acc2[mb][nb][i] * inv;
          const int64_t idx = orig * a.d_e + col0 + nb * 16 + r;
          a.a_out[idx] = f2bf(o);
          if (a.a_save) a.a_save[idx] = o;
        }
      }
    }
  __syncthreads();
}

template <int NBV>
__global__ __launch_bounds__(512, 1) void seg_group_kernel(SegGroupArgs a) {
  __shared__ uint16_t s_x[2][kGT * kXS];
  __shared__ uint16_t s_p[kGT * kPS];
  __shared__ uint16_t s_v[kGW][kVR * kVS];
  __shared__ float s_red[2][kGW][kGT];
  if (a.header[0] != 0) return;
  const int n_items = a.header[3];
  const int G = gridDim.x;
  const int vb = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8
                              : blockIdx.x;
  uint16_t* my_v = s_v[threadIdx.x >> 6];
  for (int item = vb; item < n_items; item += G) {
    const int2 im = a.gitem_map[item];
    const int s = im.x, tile = im.y;
    const int t_begin = a.seg_tok_start[s];
    const int m = a.seg_tok_start[s + 1] - t_begin;
    const int tok0 = t_begin + tile * kGT;
    const int mcount = min(kGT, m - tile * kGT);
    const int n = a.seg_n[s];
    const int64_t rowbase = a.seg_row_off[s];
#define L3_ITEM(MB, NBW) \
  group_item<MB, NBW, NBV>(a, tok0, mcount, n, rowbase, s_x, s_p, my_v, s_red)
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
  }
}

bool seg_group_ok(int d, int d_e) {
  // d: whole 16-step K rings (32 columns a step); d_e: whole 16-column
  // value blocks per wave
  return d % 512 == 0 && d_e % 128 == 0 && d_e <= kGW * kCPWMax;
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
