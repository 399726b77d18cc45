// Internal declarations shared by the C-ABI layer (api.cpp) and the HIP
// kernels. Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "l3.h"

namespace l3 {

// Tokens handled by one work item of the segment forward wave kernel (the M
// size of one 16x16 MFMA block).
constexpr int kTokTile = 16;
// Most rows of one id handled by one wave-kernel work item; ids with more
// rows are split into row chunks merged by the combine kernel.
constexpr int kWaveMaxRows = 128;
// Tokens handled by one item of the group kernel (ids with many rows).
constexpr int kGroupTok = 64;
// Ids of the group kernel with more than kGroupTok tokens are cut into
// items of this many tokens (K_t and V_t are read once per item).
constexpr int kHotTok = 128;
// Largest batch sorted by the single-workgroup plan kernel (measured: at
// 4096 tokens both paths take 0.053 ms, at 8192 the radix path 0.055 ms
// against 0.10).
constexpr int kSmallPlanMax = 4096;
// Elements per block of the multi-kernel radix sort.
constexpr int kSortTile = 1024;

// Bits of the device-side validation word of a plan.
constexpr int kBadId = 1;
constexpr int kBadCount = 2;
constexpr int kBadStage = 4;  // staged rows exceed the staging tables

// Device arrays of one plan, carved out of the caller's plan workspace.
struct PlanDev {
  int32_t* header;          // [0] status bits, [1] S, [2] wave items,
                            // [3] group items, [4], [5], [7], [9] group-kernel
                            // work queues (zero between launches),
                            // [8] wave items of every segment,
                            // [16 + x] 128-token items of XCD x's list,
                            // [24 + x] XCD x's queue of them (zero between
                            // launches); kHeaderInts in all
  int32_t* perm;            // [B] token index at sorted position
  int32_t* sorted_ids;      // [B]
  int32_t* seg_id;          // [B]
  int32_t* seg_tok_start;   // [B+1]
  int64_t* seg_row_off;     // [B]
  int32_t* seg_n;           // [B]
  int32_t* seg_item_start;  // [B+1] wave items
  int32_t* seg_gitem_start; // [B+1] group items
  int32_t* keys_alt;        // [B] radix ping-pong
  int32_t* vals_alt;        // [B]
  int32_t* hist;            // [512 * ceil(B / kSortTile)] (9-bit digits)
  int32_t* blk;             // [ceil(B / kSortTile) + 1]: the first sort
                            // pass's per-tile id checks, then the tiles'
                            // segment counts
  int2* item_map;           // wave item -> (segment, index within segment)
  int2* gitem_map;          // group item -> (segment, tile within segment)
  int2* hitem_map;          // the 128-token group items only, in kXcds
                            // lists of hitem_cap(B) entries (list x at
                            // x * hitem_cap(B), any order within a list):
                            // every item of one id in the same list
  // Wave items of every segment (the training forward runs all ids through
  // the wave kernel); count in header[8]. Only filled when the group kernel
  // is enabled (else the wave items are already all of them).
  int32_t* seg_aitem_start; // [B+1]
  int2* aitem_map;
  int64_t* stage_off;       // [B] first row of each segment in staged tables
};
// Capacity of the item maps for a batch of B tokens: a segment of m tokens
// has at most ceil(m / 16) token tiles times ceil(512 / 32) row chunks.
__host__ __device__ inline int64_t wave_items_cap(int64_t B) {
  return (B / kTokTile + B + 1) * (L3_MAX_ROWS_PER_ID / 32);
}
__host__ __device__ inline int64_t group_items_cap(int64_t B) {
  return B / kGroupTok + B + 1;
}
// Ints of a plan's header (see PlanDev::header).
constexpr int kHeaderInts = 32;
// XCDs of the device: the group kernel's workgroup b runs on XCD b % kXcds
// (workgroups are dispatched to the XCDs in turn), and takes the 128-token
// items of list b % kXcds, so all the items of one busy id run on one XCD
// and share its L2 when they read K_t.
constexpr int kXcds = 8;
// Entries of one list: an id with m > kGroupTok tokens has ceil(m / kHotTok)
// <= m / kGroupTok items, so all of them, even in one list, fit.
__host__ __device__ inline int64_t hitem_cap(int64_t B) {
  return B / kGroupTok + 1;
}
// List of segment g's 128-token items: the XCDs in turn, reversed every
// other round (segments come in id order, and frequent ids have most items)
__host__ __device__ inline int hot_list_of(int g) {
  const int q = g / kXcds, r = g % kXcds;
  return (q & 1) ? kXcds - 1 - r : r;
}

struct PlanParams {
  const int32_t* ids;
  const int64_t* offsets;
  int64_t vocab, rows;
  int B;
  int k_max;
  int chunk_rows;  // rows of one forward work item (multiple of 16)
  int group_min_rows;  // ids with this many rows use the group kernel (0: off)
};

// Arguments of the segment forward kernel (softmax-attention of each token
// over its id's rows).
struct SegFwdArgs {
  const int32_t* header;
  const int32_t* perm;
  const int32_t* seg_tok_start;
  const int64_t* seg_row_off;
  const int32_t* seg_n;
  const int32_t* seg_item_start;
  const int2* item_map;
  int count_slot;   // header slot holding the number of items
  const void* x;
  const void* K;
  const void* V;
  int d, d_e;
  int chunk_rows;   // rows per work item
  int nch_max;      // ceil(k_max / chunk_rows)
  void* a_out;      // [B x d_e] activation dtype, original token order
  float* a_save;    // [B x d_e] float32 or NULL
  float* part;      // [B x nch_max x d_e] partial sums (split rows only)
  float* part_ml;   // [B x nch_max x 2] partial (max, sum)
};

struct CombineArgs {
  int group_min_rows;
  const int32_t* header;
  const int32_t* perm;
  const int32_t* seg_tok_start;
  const int32_t* seg_n;
  int B, d_e, chunk_rows, nch_max;
  const float* part;
  const float* part_ml;
  void* a_out;
  float* a_save;
};

// Generic strided GEMM: C[m, n] = sum_k A(m, k) * B(k, n) with
//   A(m, k) = k < K1 ? A1[m*a1_m + k*a1_k] : A2[m*a2_m + (k-K1)*a2_k]
//   B(k, n) = Bm[k*b_k + n*b_n]
// float32 accumulation, fixed summation order.
struct GemmArgs {
  const void* A1;
  const void* A2;
  int64_t a1_m, a1_k, a2_m, a2_k;
  int K1;
  const void* Bm;
  int64_t b_k, b_n;
  void* C;
  int64_t c_m;
  int M, N, K;
  const int32_t* header;  // plan status word (kernel does nothing if set)
  // generic kernel only: split of K over workgroups, partial M x N float32
  // products in part (nsplit of them), summed in order by a second kernel
  float* part = nullptr;
  int nsplit = 1;
  // 256 x 256 kernel only: LayerNorm folded into the GEMM that consumes
  // its output (h = gamma * (u - mean) * rstd + beta, then y = [h ; x] W^T):
  //   producer (u = a W_up^T): ln_stats_out[m * (N / 256) + t] = (mean, M2)
  //     of row m over the 256 columns of tile t (float32 pairs);
  //   consumer (y): for k < K1 the B operand is B1 (row stride b1_n), W with
  //     gamma folded in; ln_rows[m] = (rstd, -mean * rstd) of row m and
  //     ln_c12[n] = (c1, c2) the folded column sums; after the k < K1 part,
  //     acc = rstd * acc - mean * rstd * c1 + c2.
  const void* B1 = nullptr;
  int64_t b1_n = 0;
  // 256 x 256 kernel: for k >= K1 read Bm's column k - K1 instead of k
  // (B1 then holds the k < K1 part, as for A1 / A2)
  int b2_rel = 0;
  float* ln_stats_out = nullptr;
  const float* ln_rows = nullptr;
  const float* ln_c12 = nullptr;
  // 256 x 256 kernel, quadratic-form epilogue (gemm_nt_256_quad_launch):
  // ln_stats_out[m * (N / 256) + t] = (sum_n Q[m, n] * C[m, n], 0) over the
  // 256 columns n of tile t, Q bf16 with row stride ln_quad_lda; C itself
  // is not written.
  const uint16_t* ln_quad_a = nullptr;
  int64_t ln_quad_lda = 0;
};

// Row statistics of the fold from the producer's partials.
struct LnRowsArgs {
  const int32_t* header;
  const float* part;   // [B x nparts] (mean, M2) pairs over 256 columns
  int nparts, B, d;
  float eps;
  float* rows;         // [B] (rstd, -mean * rstd) pairs
  // quad: the parts' first members add up to sum_j (u_j - mean)^2 itself
  // (the quadratic-form epilogue); rows = (rstd, 0)
  int quad = 0;
};

// Fold of LayerNorm's affine into the first K1 columns of W_mix (rows of W
// have stride w_n): W1[n, k] = bf16(W[n, k] * gamma[k]) for k < d,
// c12[n] = (sum_k W1[n, k], sum_k W[n, k] * beta[k]) in float32.
struct LnFoldArgs {
  const int32_t* header;
  const uint16_t* W;
  int64_t w_n;
  const uint16_t* gamma;
  const uint16_t* beta;
  int n, d;
  uint16_t* W1;     // [n x d] bf16, or NULL: c12 only
  float* c12;       // [n x 2]
  // split: W1 rows [n x 2d], the bf16 product at [0, d) and the bf16
  // rounding residual at [d, 2d); c1 = 0
  int split = 0;
};

// LayerNorm of float32 rows (one wave per row).
struct LnArgs {
  const int32_t* header;
  const float* U;
  const void* gamma;
  const void* beta;
  int B, d;
  float eps;
  void* h;        // [B x d] activation dtype
  float* h_save;  // [B x d] or NULL
  float* uhat_save;
  float* rstd_save;
};

enum ElemType { kF32 = L3_F32, kBF16 = L3_BF16 };

// ---- launchers (return the first HIP error) -------------------------------
hipError_t plan_launch(const PlanDev& pd, const PlanParams& pp,
                       hipStream_t s);
hipError_t seg_fwd_launch(const SegFwdArgs& a, int dtype, int B, int items_ub,
                          hipStream_t s);
hipError_t seg_combine_launch(const CombineArgs& a, int dtype, hipStream_t s);

// Group kernel: one workgroup per (id, tile of 64 tokens), all of the id's
// rows; bf16 only, d % 64 == 0, d_e % 128 == 0, d_e <= 512.
struct SegGroupArgs {
  const int32_t* header;
  const int32_t* perm;
  const int32_t* seg_tok_start;
  const int64_t* seg_row_off;
  const int32_t* seg_n;
  const int32_t* seg_gitem_start;
  const int2* gitem_map;
  const int2* hitem_map;   // kXcds lists of hcap entries
  int hcap;
  int* work;        // header + 4: [0] queue of the 64-token pass, [1]
                    // finished workgroups, [5] queue of the wave-item pass,
                    // [20 + x] queue of XCD x's 128-token items
  const uint16_t* x;
  const uint16_t* K;
  const uint16_t* V;
  int d, d_e;
  uint16_t* a_out;  // [B x d_e] bf16, original token order
  float* a_save;    // [B x d_e] float32 or NULL
  // wave items taken in a last pass (header NULL: none); bf16 inference
  SegFwdArgs wave;
};
// Staging of the batch's rows from host-resident tables (stage.hip).
struct StageArgs {
  int32_t* header;
  const int32_t* seg_n;
  int64_t* seg_row_off;   // rewritten to the staged offsets
  int64_t* stage_off;
  int d, d_e, elem;       // row widths, element bytes
  int64_t stage_rows;     // capacity of K_stage / V_stage in rows
  const uint8_t* K_host;
  const uint8_t* V_host;
  uint8_t* K_stage;
  uint8_t* V_stage;
};
hipError_t stage_rows_launch(const StageArgs& a, int S_ub, hipStream_t s);

bool seg_group_ok(int d, int d_e);
hipError_t seg_group_launch(const SegGroupArgs& a, int items_ub,
                            hipStream_t s);
hipError_t gemm_launch(const GemmArgs& g, int a_type, int b_type, int c_type,
                       hipStream_t s, float* part = nullptr,
                       int64_t part_floats = 0);
hipError_t gemm_nt_mfma_launch(const GemmArgs& g, int c_type, hipStream_t s,
                               float* part = nullptr,
                               int64_t part_floats = 0);
bool gemm_nt_mfma_ok(const GemmArgs& g);
// The 256 x 256 tile kernel (the only one with the LayerNorm fold); the
// launcher above takes it for these shapes when no split-K buffer is given.
bool gemm_nt_256_ok(const GemmArgs& g);
hipError_t ln_fold_launch(const LnFoldArgs& a, hipStream_t s);
// Centred, transposed bf16 hi | lo copy of W (rows x cols, bf16):
// T[c, r] = hi, T[c, rows + r] = hi, T[c, 2 rows + r] = lo of
// W[r, c] - mean_r W[r, c] (T is [cols x 3 rows]); mean is scratch of
// cols * ceil(rows / 64) floats (column sums per block of 64 rows).
// ln_fold_launch(fa) and center_split_t_launch(fa.header, W, ...) with the
// fold and the column sums in one launch (they are independent); fa.W1 may
// be NULL (c12 only). With T2, also T2[c, r] = hi, T2[c, rows + r] = lo of
// gamma[r] (W[r, c] - mean_r W[r, c]) (T2 is [cols x 2 rows]).
hipError_t fold_prep_launch(const LnFoldArgs& fa, const uint16_t* W,
                            int rows, int cols, float* mean, uint16_t* T,
                            const uint16_t* gamma, uint16_t* T2,
                            hipStream_t s);
hipError_t center_split_t_launch(const int32_t* header, const uint16_t* W,
                                 int rows, int cols, float* mean, uint16_t* T,
                                 hipStream_t s);
// Centred row-major bf16 hi | lo copy of W (rows x cols, bf16): out[r, c] =
// hi, out[r, cols + c] = lo of W[r, c] - mean_r W[r, c] (out is
// [rows x 2 cols]); mean as above.
hipError_t center_split_launch(const int32_t* header, const uint16_t* W,
                               int rows, int cols, float* mean, uint16_t* out,
                               hipStream_t s);
hipError_t gemm_nt_256_quad_launch(const GemmArgs& g, hipStream_t s);
hipError_t ln_rows_launch(const LnRowsArgs& a, hipStream_t s);
hipError_t ln_launch(const LnArgs& a, int dtype, hipStream_t s);
// u = A B^T (float32, into ln.U unless fused), then LayerNorm rows into ln.h
hipError_t gemm_ln_launch(const GemmArgs& g, const LnArgs& ln, int dtype,
                          hipStream_t s, float* part, int64_t part_floats);

struct BwdArgs {
  const int32_t* header;
  const int32_t* perm;
  const int32_t* seg_tok_start;
  const int64_t* seg_row_off;
  const int32_t* seg_n;
  int B, d, d_e;
  const void* x;
  const void* K;
  const void* V;
  const void* gamma;
  const float* uhat;   // saved
  const float* rstd;   // saved
  const float* dH;     // [B x d]
  float* dU;           // [B x d]
  const float* dA;     // [B x d_e]
  float* dx;           // [B x d], holds dX_b on entry
  float* dK;
  float* dV;
  float* dgamma;
  float* dbeta;
  int64_t rows;
  // segment backward: the training forward's work items (token tile, row
  // chunk) and two [B x kst] float32 arrays for p and dS (sorted order)
  const int2* item_map;
  int count_slot;
  int chunk_rows;
  int kst;             // row stride of Pbuf / DSbuf: k_max rounded up to 16
  float* Pbuf;
  float* DSbuf;
  float* ln_part;      // [ceil(B / 256) x 2 x d] LayerNorm column partials
  // (segment, 64-row block) pairs of the column pass, and their count
  int2* rows_map;      // [B x ceil(kst / 64)] at most
  int* rows_count;
  // (first row, rows <= 64) pieces of the absent ids' rows, and their count
  int2* zero_map;      // [rows / 64 + B + 2] at most
  int* zero_count;
  // per (token, row chunk) softmax statistics (M, L, Q, -) of the chunked
  // tile pass; NULL: one wave walks each tile's chunks
  float4* chunk_stats; // [B x cs_stride]
  int cs_stride;       // row chunks of the longest id
  // the plan's 64-token items (ids with at least group_min_rows rows; 0:
  // none) for the dX_att pass
  const int2* gitem_map = nullptr;
  int group_min_rows = 0;
};
// Zeroes dK, dV rows of the ids absent from the batch (d, d_e multiples of
// 4); items_ub bounds the number of 64-row pieces.
hipError_t zero_absent_launch(const BwdArgs& a, int64_t items_ub,
                              hipStream_t s);
hipError_t fill_zero_launch(float* p, int64_t n, hipStream_t s);
// dst [cols x rows] (row stride ldd, default rows) = transpose of src
// [rows x cols] (row stride ld), bf16.
hipError_t transpose_bf16_launch(const int32_t* header, const uint16_t* src,
                                 int64_t ld, int rows, int cols,
                                 uint16_t* dst, hipStream_t s,
                                 int64_t ldd = 0);
// Float32 [n] (n a multiple of 4 for whole vectors; any n works) to its
// bf16 hi and lo halves: hi = bf16(v), lo = bf16(v - hi).
hipError_t split_bf16_launch(const int32_t* header, const float* src,
                             int64_t n, uint16_t* hi, uint16_t* lo,
                             hipStream_t s);
// Transpose of float32 src [rows x cols] as bf16 hi / lo halves: dst row c
// (stride ldd, default 2 rows) holds hi at r, lo at lo_off + r (default
// rows) and, if hi2_off >= 0, hi again at hi2_off + r.
hipError_t transpose_split_launch(const int32_t* header, const float* src,
                                  int64_t ld, int rows, int cols,
                                  uint16_t* dst, hipStream_t s,
                                  int64_t ldd = 0, int64_t lo_off = 0,
                                  int64_t hi2_off = -1);
// The 256 x 256 bf16 kernel with K split over workgroups into float32
// partials (part), reduced in order into C (float32). hipErrorInvalidValue
// if the shape rules of the 256 x 256 kernel do not hold.
hipError_t gemm_nt_256_splitk_launch(const GemmArgs& g, hipStream_t s,
                                     float* part, int64_t part_floats,
                                     int max_split = 16,
                                     int c_type = kF32);
// Two independent products of that form in one launch (and their sums in
// one more): a's C as bf16, b's as the bf16 hi (C) | lo (b_lo) pair of its
// float32 sum, with the K shares the single launcher would choose.
// hipErrorInvalidValue (nothing launched) if the shapes do not allow it.
hipError_t gemm_nt_256_splitk_pair_launch(const GemmArgs& a, int max_a,
                                          const GemmArgs& b, int max_b,
                                          uint16_t* b_lo, float* part,
                                          int64_t part_floats, hipStream_t s);
hipError_t ln_bwd_launch(const BwdArgs& a, int dtype, hipStream_t s);
hipError_t seg_bwd_launch(const BwdArgs& a, int dtype, int items_ub,
                          int S_ub, hipStream_t s);

}  // namespace l3
