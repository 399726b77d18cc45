// C-ABI layer of libl3: argument checks, workspace carving and the launch
// sequence of the plan, forward and backward passes on the caller's stream.
// Nothing here allocates device memory or synchronises the stream on the
// plan / forward / backward path. No C++ exception leaves an extern "C"
// function.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "l3.h"
#include "l3_internal.h"

using namespace l3;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline bool aligned(const void* p) {
  return reinterpret_cast<uintptr_t>(p) % kAlign == 0;
}

// Bump allocator over a caller workspace (base == nullptr only measures).
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    off = align_up(off);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
  size_t bytes() const { return align_up(off); }
};

enum Stage {
  ST_PLAN,
  ST_SEG,
  ST_COMBINE,
  ST_UP,
  ST_LN,
  ST_MIX,
  ST_BWD_MIX,
  ST_BWD_LN,
  ST_BWD_UP,
  ST_BWD_SEG,
  ST_GROUP,
  ST_WFOLD,
  ST_UP_QUAD,
  ST_MIX_UP,
  ST_COUNT
};
const char* const kStageNames[ST_COUNT] = {
    "plan",        "seg_fwd", "seg_combine",   "up_proj", "layernorm",
    "mix_proj",    "bwd_mix", "bwd_layernorm", "bwd_up",  "bwd_seg",
    "seg_group",   "weight_fold", "up_quad", "mix_up_proj"};

bool debug_sync() {
  static const bool on = [] {
    const char* e = std::getenv("L3_DEBUG_SYNC");
    return e && e[0] && e[0] != '0';
  }();
  return on;
}

inline size_t elem_bytes(int dtype) { return dtype == L3_BF16 ? 2 : 4; }

l3_status check_desc(const l3_desc* d) {
  if (!d) return L3_ERR_NULL;
  if (d->dtype != L3_F32 && d->dtype != L3_BF16) return L3_ERR_DTYPE;
  if (d->y_dtype != L3_F32 && d->y_dtype != L3_BF16) return L3_ERR_DTYPE;
  if (d->vocab < 1 || d->rows < 1) return L3_ERR_SHAPE;
  if (d->d < 64 || d->d % 64 != 0 || d->d > 4096) return L3_ERR_SHAPE;
  if (d->d_k != d->d) return L3_ERR_SHAPE;
  if (d->d_e < 64 || d->d_e % 64 != 0 || d->d_e > 4096) return L3_ERR_SHAPE;
  if (d->k_max < 1 || d->k_max > L3_MAX_ROWS_PER_ID) return L3_ERR_SHAPE;
  if (!(d->ln_eps >= 0.0f) || !std::isfinite(d->ln_eps)) return L3_ERR_SHAPE;
  if (d->vocab > (int64_t(1) << 31) - 2) return L3_ERR_SHAPE;
  return L3_OK;
}

// Rows of one wave-kernel work item: small batches split an id's rows
// finely so that enough wavefronts stream them; otherwise an item takes up
// to kWaveMaxRows rows (ids with more rows are split into chunks, or go to
// the group kernel in large bf16 batches).
int chunk_rows_for(int64_t B, int k_max) {
  int ch = B <= 256 ? 32 : kWaveMaxRows;
  int kp = 16;
  while (kp < k_max) kp <<= 1;
  return ch < kp ? ch : kp;
}
int nch_for(int64_t B, int k_max) {
  const int ch = chunk_rows_for(B, k_max);
  return (k_max + ch - 1) / ch;
}

// Large bf16 batches send ids with at least this many rows to the group
// kernel (a workgroup per 64-token tile streams the id's whole K_t, V_t
// slice); 0 disables it. Small batches keep every id on the wave kernel,
// whose row chunks spread one id over many wavefronts.
constexpr int kGroupMinRows = 128;
// Whether folding W_up into W_mix pays: the flops it saves (the W_up GEMM
// and d - d_e of W_mix's K, less the a G product) must reach 1e11, about
// twice what the per-call weight products (~0.1 ms) cost at the GEMMs' rate.
bool fuse_up_pays(int64_t B, int64_t d, int64_t de) {
  const double per_row = 2.0 * d * de + 2.0 * d * (d - de) - 4.0 * de * de;
  return static_cast<double>(B) * per_row >= 1e11;
}
int group_min_rows_for(const l3_desc& d, int64_t B) {
  return (d.dtype == L3_BF16 && B > 2048 && seg_group_ok(d.d, d.d_e))
             ? kGroupMinRows
             : 0;
}

PlanDev carve_plan(Carver& c, int64_t B) {
  const size_t nb = static_cast<size_t>(B);
  const size_t nblk = (nb + kSortTile - 1) / kSortTile;
  PlanDev p;
  p.header = c.take<int32_t>(kHeaderInts);
  p.perm = c.take<int32_t>(nb);
  p.sorted_ids = c.take<int32_t>(nb);
  p.seg_id = c.take<int32_t>(nb);
  p.seg_tok_start = c.take<int32_t>(nb + 1);
  p.seg_row_off = c.take<int64_t>(nb);
  p.seg_n = c.take<int32_t>(nb);
  p.seg_item_start = c.take<int32_t>(nb + 1);
  p.seg_gitem_start = c.take<int32_t>(nb + 1);
  p.keys_alt = c.take<int32_t>(nb);
  p.vals_alt = c.take<int32_t>(nb);
  p.hist = c.take<int32_t>(512 * nblk);
  p.blk = c.take<int32_t>(nblk + 1);
  p.item_map = c.take<int2>(static_cast<size_t>(wave_items_cap(B)));
  p.gitem_map = c.take<int2>(static_cast<size_t>(group_items_cap(B)));
  p.hitem_map = c.take<int2>(static_cast<size_t>(kXcds * hitem_cap(B)));
  p.seg_aitem_start = c.take<int32_t>(nb + 1);
  p.aitem_map = c.take<int2>(static_cast<size_t>(wave_items_cap(B)));
  p.stage_off = c.take<int64_t>(nb);
  return p;
}

struct SaveBufs {
  float* a32;   // [B x d_e]
  float* uhat;  // [B x d]
  float* h32;   // [B x d]
  float* rstd;  // [B]
};
SaveBufs carve_save(Carver& c, const l3_desc& d, int64_t B) {
  SaveBufs s;
  s.a32 = c.take<float>(B * d.d_e);
  s.uhat = c.take<float>(B * d.d);
  s.h32 = c.take<float>(B * d.d);
  s.rstd = c.take<float>(B);
  return s;
}

// Room for split-K partials: eight d x max(d, d_e) products, at most 16 MB.
int64_t gpart_floats_for(const l3_desc& d) {
  const int64_t w = static_cast<int64_t>(d.d) * (d.d > d.d_e ? d.d : d.d_e);
  const int64_t f = 8 * w;
  return f < (int64_t(1) << 22) ? f : (int64_t(1) << 22);
}

// Split-K partials of the bf16 weight-gradient GEMMs of dW_mix (d x d
// outputs on 256 x 256 tiles, up to 16 shares so that about 256 workgroups
// run); 0 where those GEMMs do not apply.
int64_t splitk_floats_for(const l3_desc& d) {
  if (d.dtype != L3_BF16 || d.d % 256 != 0 || d.d < 1024) return 0;
  const int64_t tiles = static_cast<int64_t>(d.d / 256) * (d.d / 256);
  int64_t ns = (256 + tiles - 1) / tiles;
  if (ns > 16) ns = 16;
  return ns > 1 ? ns * d.d * d.d : 0;
}

struct FwdBufs {
  void* a_act;  // [B x d_e] dtype
  float* U;     // [B x d]
  void* h_act;  // [B x d] dtype
  float* part;
  float* part_ml;
  float* gpart;  // split-K partial products of small-batch GEMMs
  int64_t gpart_floats;
  // training, bf16: the float32 aggregate as bf16 hi | lo [B x d_e] each
  uint16_t* a_hi;
  uint16_t* a_lo;
  // bf16: W_up with its columns centred, as bf16 hi | lo [d x 2 d_e], and
  // the column sums it is built from [ceil(d / 64) x d_e]
  uint16_t* wc;
  float* wc_part;
};
FwdBufs carve_fwd(Carver& c, const l3_desc& d, int64_t B) {
  FwdBufs f;
  const size_t es = elem_bytes(d.dtype);
  f.a_act = c.take<char>(B * d.d_e * es);
  f.U = c.take<float>(B * d.d);
  f.h_act = c.take<char>(B * d.d * es);
  const int nch = nch_for(B, d.k_max);
  if (nch > 1) {
    f.part = c.take<float>(B * nch * d.d_e);
    f.part_ml = c.take<float>(B * nch * 2);
  } else {
    f.part = nullptr;
    f.part_ml = nullptr;
  }
  // small batches split K of the projections (few output tiles)
  f.gpart_floats = B < 1024 ? gpart_floats_for(d) : 0;
  f.gpart = f.gpart_floats ? c.take<float>(f.gpart_floats) : nullptr;
  const bool b16 = d.dtype == L3_BF16;
  const size_t ae = static_cast<size_t>(B) * d.d_e;
  f.a_hi = b16 ? c.take<uint16_t>(ae) : nullptr;
  f.a_lo = b16 ? c.take<uint16_t>(ae) : nullptr;
  const size_t wce = static_cast<size_t>(d.d) * 2 * d.d_e;
  f.wc = b16 ? c.take<uint16_t>(wce) : nullptr;
  f.wc_part = b16 ? c.take<float>(static_cast<size_t>((d.d + 63) / 64) * d.d_e)
                  : nullptr;
  return f;
}

struct BwdBufs {
  float* dH;
  float* dU;
  float* dA;
  float* P;   // [B x bwd_kst] softmax weights, sorted token order
  float* dS;  // [B x bwd_kst] score gradients
  float* ln_part;  // [ceil(B / 256) x 2 x d] dgamma / dbeta partials
  float* gpart;    // split-K partial products of the weight gradients
  int64_t gpart_floats;
  uint16_t* wmixT;  // [2d x d] W_mix transposed (bf16 only)
  uint16_t* dyT;    // [d x B] dY transposed (bf16 only)
  uint16_t* xT;     // [d x B] x transposed (bf16 only)
  uint16_t* hT;     // [d x 2B] saved h transposed, bf16 hi | lo (bf16 only)
  int2* rows_map;   // segment backward's column-pass work list
  int* rows_count;
  int2* zero_map;   // 64-row pieces of the absent ids' rows
  int* zero_count;
  float4* chunk_stats;  // [B x ceil(k_max / 32)] (bf16 only)
};
int64_t zero_items_for(const l3_desc& d, int64_t B) {
  return d.rows / 64 + B + 2;
}

// Row stride of the segment backward's p / dS arrays: k_max rounded up to
// its 64-row blocks.
int bwd_kst(const l3_desc& d) { return (d.k_max + 63) / 64 * 64; }
BwdBufs carve_bwd(Carver& c, const l3_desc& d, int64_t B) {
  BwdBufs b;
  b.dH = c.take<float>(B * d.d);
  b.dU = c.take<float>(B * d.d);
  b.dA = c.take<float>(B * d.d_e);
  b.P = c.take<float>(B * bwd_kst(d));
  b.dS = c.take<float>(B * bwd_kst(d));
  b.ln_part = c.take<float>((B + 255) / 256 * 2 * d.d);
  b.gpart_floats = std::max(gpart_floats_for(d), splitk_floats_for(d));
  b.gpart = c.take<float>(b.gpart_floats);
  const bool b16 = d.dtype == L3_BF16;
  b.wmixT = b16 ? c.take<uint16_t>(static_cast<size_t>(2) * d.d * d.d)
                : nullptr;
  b.dyT = b16 ? c.take<uint16_t>(static_cast<size_t>(B) * d.d) : nullptr;
  b.xT = b16 ? c.take<uint16_t>(static_cast<size_t>(B) * d.d) : nullptr;
  b.hT = b16 ? c.take<uint16_t>(static_cast<size_t>(2) * B * d.d) : nullptr;
  b.rows_map = c.take<int2>(static_cast<size_t>(B) *
                            ((bwd_kst(d) + 63) / 64));
  b.rows_count = c.take<int>(64);
  b.zero_map = c.take<int2>(static_cast<size_t>(zero_items_for(d, B)));
  b.zero_count = c.take<int>(64);
  // row chunks are at least 32 rows
  b.chunk_stats = b16 ? c.take<float4>(static_cast<size_t>(B) *
                                       ((d.k_max + 31) / 32))
                      : nullptr;
  return b;
}

size_t plan_bytes(int64_t B) {
  Carver c(nullptr);
  carve_plan(c, B);
  return c.bytes();
}
size_t save_bytes_for(const l3_desc& d, int64_t B) {
  Carver c(nullptr);
  carve_save(c, d, B);
  return c.bytes();
}
size_t fwd_bytes_for(const l3_desc& d, int64_t B) {
  Carver c(nullptr);
  carve_fwd(c, d, B);
  return c.bytes();
}
size_t bwd_bytes_for(const l3_desc& d, int64_t B) {
  Carver c(nullptr);
  carve_bwd(c, d, B);
  return c.bytes();
}
size_t scratch_bytes_for(const l3_desc& d, int64_t B) {
  size_t f = fwd_bytes_for(d, B), b = bwd_bytes_for(d, B);
  return f > b ? f : b;
}

}  // namespace

struct l3_plan_s {
  l3_desc desc;
  int64_t B = 0;
  int64_t capacity = 0;  // largest B the workspace holds
  int chunk_rows = 32;
  int nch_max = 1;
  int group_min_rows = 0;
  PlanDev dev;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  bool timing = false;
  struct Ev {
    hipEvent_t a, b;
    int stage;
  };
  std::vector<Ev> events;
  // save workspaces written by saving forwards since the last (re)plan: one
  // plan can serve several layers, each with its own save workspace
  std::vector<const void*> saved;
  // l3_stage_rows pointed the segments at staged tables (inference only)
  bool staged = false;
  // pinned host mirror of the segments for l3_stage_rows_dma (made on
  // first use): S, then (row offset, rows) per segment, then staged offsets
  int64_t* host_seg = nullptr;
  size_t host_seg_count = 0;
};

namespace {

// Records a pair of events around one stage when timing is on.
struct StageTimer {
  l3_plan_s* p;
  int stage;
  hipStream_t s;
  hipEvent_t a = nullptr, b = nullptr;
  bool on;
  StageTimer(l3_plan_s* plan, int st, hipStream_t stream)
      : p(plan), stage(st), s(stream), on(plan->timing) {
    if (on) {
      if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
        on = false;
        return;
      }
      hipEventRecord(a, s);
    }
  }
  ~StageTimer() {
    if (on) {
      hipEventRecord(b, s);
      p->events.push_back({a, b, stage});
    }
  }
};

l3_status finish(l3_plan_s* p, hipError_t e, hipStream_t s) {
  if (e != hipSuccess) return L3_ERR_HIP;
  if (debug_sync()) {
    if (hipStreamSynchronize(s) != hipSuccess) return L3_ERR_HIP;
    if (p && p->B > 0) {
      int32_t h = 0;
      if (hipMemcpy(&h, p->dev.header, sizeof(h), hipMemcpyDeviceToHost) !=
          hipSuccess)
        return L3_ERR_HIP;
      if (h & kBadId) return L3_ERR_TOKEN_RANGE;
      if (h & kBadCount) return L3_ERR_COUNT;
      if (h & kBadStage) return L3_ERR_WORKSPACE;
    }
  }
  return L3_OK;
}

l3_status do_plan(l3_plan_s* p, const int32_t* ids, int64_t B,
                  const int64_t* offsets, hipStream_t s) {
  if (B < 0) return L3_ERR_SHAPE;
  if (B > p->capacity) return L3_ERR_WORKSPACE;
  if (B > 0 && (!ids || !offsets)) return L3_ERR_NULL;
  p->B = B;
  p->saved.clear();
  p->staged = false;
  p->chunk_rows = chunk_rows_for(B, p->desc.k_max);
  p->nch_max = nch_for(B, p->desc.k_max);
  p->group_min_rows = group_min_rows_for(p->desc, B);
  Carver c(p->ws);
  p->dev = carve_plan(c, B);
  if (B == 0) return L3_OK;
  PlanParams pp;
  pp.ids = ids;
  pp.offsets = offsets;
  pp.vocab = p->desc.vocab;
  pp.rows = p->desc.rows;
  pp.B = static_cast<int>(B);
  pp.k_max = p->desc.k_max;
  pp.chunk_rows = p->chunk_rows;
  pp.group_min_rows = p->group_min_rows;
  hipError_t e;
  {
    StageTimer t(p, ST_PLAN, s);
    e = plan_launch(p->dev, pp, s);
  }
  return finish(p, e, s);
}

}  // namespace

extern "C" {

const char* l3_status_str(l3_status st) {
  switch (st) {
    case L3_OK: return "ok";
    case L3_ERR_NULL: return "a required pointer is NULL";
    case L3_ERR_SHAPE: return "unsupported or inconsistent sizes";
    case L3_ERR_DTYPE: return "unknown element type";
    case L3_ERR_WORKSPACE: return "workspace too small";
    case L3_ERR_HIP: return "HIP runtime error";
    case L3_ERR_TOKEN_RANGE: return "token id outside [0, vocab)";
    case L3_ERR_COUNT: return "an id owns 0 or more than k_max rows, or rows outside the table";
    case L3_ERR_STATE: return "call out of order";
    default: return "unknown status";
  }
}

const char* l3_stage_name(int stage) {
  return (stage >= 0 && stage < ST_COUNT) ? kStageNames[stage] : nullptr;
}

l3_status l3_workspace_size(const l3_desc* desc, int64_t max_tokens,
                            size_t* plan_ws, size_t* save_ws,
                            size_t* scratch_ws) {
  l3_status st = check_desc(desc);
  if (st != L3_OK) return st;
  if (max_tokens < 0 || max_tokens >= (int64_t(1) << 31)) return L3_ERR_SHAPE;
  if (plan_ws) *plan_ws = plan_bytes(max_tokens);
  if (save_ws) *save_ws = save_bytes_for(*desc, max_tokens);
  if (scratch_ws) {
    // the forward's split-row partials depend on the batch size actually
    // planned; take the largest need over every batch up to max_tokens
    size_t m = scratch_bytes_for(*desc, max_tokens);
    const int64_t probes[2] = {256, 2048};
    for (int64_t b : probes) {
      if (b < max_tokens) {
        size_t v = scratch_bytes_for(*desc, b);
        if (v > m) m = v;
      }
    }
    *scratch_ws = m;
  }
  return L3_OK;
}

l3_status l3_plan(const l3_desc* desc, const int32_t* ids, int64_t B,
                  const int64_t* offsets, void* plan_ws, size_t plan_ws_bytes,
                  void* stream, l3_plan_t* out) {
  try {
    if (!out) return L3_ERR_NULL;
    *out = nullptr;
    l3_status st = check_desc(desc);
    if (st != L3_OK) return st;
    if (B < 0 || B >= (int64_t(1) << 31)) return L3_ERR_SHAPE;
    if (!plan_ws) return L3_ERR_NULL;
    if (plan_ws_bytes < plan_bytes(B) || !aligned(plan_ws))
      return L3_ERR_WORKSPACE;
    // capacity: the largest batch whose plan fits this workspace
    int64_t lo = B, hi = (int64_t(1) << 31) - 1;
    while (lo < hi) {
      int64_t mid = lo + (hi - lo + 1) / 2;
      if (plan_bytes(mid) <= plan_ws_bytes)
        lo = mid;
      else
        hi = mid - 1;
    }
    l3_plan_s* p = new (std::nothrow) l3_plan_s();
    if (!p) return L3_ERR_HIP;
    p->desc = *desc;
    p->ws = plan_ws;
    p->ws_bytes = plan_ws_bytes;
    p->capacity = lo;
    st = do_plan(p, ids, B, offsets, static_cast<hipStream_t>(stream));
    if (st != L3_OK && st != L3_ERR_TOKEN_RANGE && st != L3_ERR_COUNT) {
      delete p;
      return st;
    }
    *out = p;
    return st;
  } catch (...) {
    return L3_ERR_HIP;
  }
}

l3_status l3_replan(l3_plan_t plan, const int32_t* ids, int64_t B,
                    const int64_t* offsets, void* stream) {
  try {
    if (!plan) return L3_ERR_NULL;
    return do_plan(plan, ids, B, offsets, static_cast<hipStream_t>(stream));
  } catch (...) {
    return L3_ERR_HIP;
  }
}

void l3_plan_release(l3_plan_t plan) {
  if (!plan) return;
  for (auto& e : plan->events) {
    hipEventDestroy(e.a);
    hipEventDestroy(e.b);
  }
  if (plan->host_seg) (void)hipHostFree(plan->host_seg);
  delete plan;
}

int64_t l3_plan_tokens(l3_plan_t plan) { return plan ? plan->B : -1; }

l3_status l3_plan_check(l3_plan_t plan, void* stream) {
  if (!plan) return L3_ERR_NULL;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess)
    return L3_ERR_HIP;
  if (plan->B == 0) return L3_OK;
  int32_t h = 0;
  if (hipMemcpy(&h, plan->dev.header, sizeof(h), hipMemcpyDeviceToHost) !=
      hipSuccess)
    return L3_ERR_HIP;
  if (h & kBadId) return L3_ERR_TOKEN_RANGE;
  if (h & kBadCount) return L3_ERR_COUNT;
  if (h & kBadStage) return L3_ERR_WORKSPACE;
  return L3_OK;
}

namespace {
// The device address of memory the GPU may read: pinned host memory known
// to HIP (its mapped address), or device / managed memory (itself). Plain
// pageable host memory is refused (the copy kernel would fault on it).
bool device_readable(const void* p, const void** out) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (attr.type == hipMemoryTypeHost) {
    *out = attr.devicePointer;
    return *out != nullptr;
  }
  if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) {
    *out = p;
    return true;
  }
  return false;
}
}  // namespace

l3_status l3_stage_rows(l3_plan_t plan, const void* K_host,
                        const void* V_host, void* K_stage, void* V_stage,
                        int64_t stage_rows, void* stream) {
  try {
    if (!plan) return L3_ERR_NULL;
    if (plan->B == 0) return L3_OK;
    if (!K_host || !V_host || !K_stage || !V_stage) return L3_ERR_NULL;
    const void* K_src = nullptr;
    const void* V_src = nullptr;
    if (!device_readable(K_host, &K_src) || !device_readable(V_host, &V_src))
      return L3_ERR_NULL;
    if (stage_rows < 0) return L3_ERR_SHAPE;
    if (plan->staged) return L3_ERR_STATE;
    const l3_desc& d = plan->desc;
    StageArgs a;
    a.header = plan->dev.header;
    a.seg_n = plan->dev.seg_n;
    a.seg_row_off = plan->dev.seg_row_off;
    a.stage_off = plan->dev.stage_off;
    a.d = d.d;
    a.d_e = d.d_e;
    a.elem = static_cast<int>(elem_bytes(d.dtype));
    a.stage_rows = stage_rows;
    a.K_host = static_cast<const uint8_t*>(K_src);
    a.V_host = static_cast<const uint8_t*>(V_src);
    a.K_stage = static_cast<uint8_t*>(K_stage);
    a.V_stage = static_cast<uint8_t*>(V_stage);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t S_ub = plan->B < d.vocab ? plan->B : d.vocab;
    hipError_t e = stage_rows_launch(a, static_cast<int>(S_ub), s);
    if (e != hipSuccess) return L3_ERR_HIP;
    plan->staged = true;
    plan->saved.clear();
    return finish(plan, e, s);
  } catch (...) {
    return L3_ERR_HIP;
  }
}

namespace {
__global__ void copy_i64_kernel(int64_t* dst, const int64_t* src, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i];
}
}  // namespace

l3_status l3_stage_rows_dma(l3_plan_t plan, const void* K_host,
                            const void* V_host, void* K_stage, void* V_stage,
                            int64_t stage_rows, void* stream) {
  try {
    if (!plan) return L3_ERR_NULL;
    if (plan->B == 0) return L3_OK;
    if (!K_host || !V_host || !K_stage || !V_stage) return L3_ERR_NULL;
    const void* K_src = nullptr;
    const void* V_src = nullptr;
    if (!device_readable(K_host, &K_src) || !device_readable(V_host, &V_src))
      return L3_ERR_NULL;
    if (stage_rows < 0) return L3_ERR_SHAPE;
    if (plan->staged) return L3_ERR_STATE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const l3_desc& d = plan->desc;
    const int64_t B = plan->B;
    const size_t need = static_cast<size_t>(4 * B + 2);
    if (plan->host_seg_count < need) {
      if (plan->host_seg) (void)hipHostFree(plan->host_seg);
      plan->host_seg = nullptr;
      plan->host_seg_count = 0;
      if (hipHostMalloc(reinterpret_cast<void**>(&plan->host_seg),
                        need * sizeof(int64_t), hipHostMallocDefault) !=
          hipSuccess)
        return L3_ERR_HIP;
      plan->host_seg_count = need;
    }
    int64_t* h = plan->host_seg;
    const PlanDev& pd = plan->dev;
    // the segments, once the plan is done (the caller orders `stream` after
    // the plan, e.g. with an event)
    int32_t hdr[2] = {0, 0};
    hipError_t e = hipMemcpyAsync(hdr, pd.header, sizeof(hdr),
                                  hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(h + 2, pd.seg_row_off, B * sizeof(int64_t),
                         hipMemcpyDeviceToHost, s);
    std::vector<int32_t> n_host(static_cast<size_t>(B));
    if (e == hipSuccess)
      e = hipMemcpyAsync(n_host.data(), pd.seg_n, B * sizeof(int32_t),
                         hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return L3_ERR_HIP;
    if (hdr[0] & kBadId) return L3_ERR_TOKEN_RANGE;
    if (hdr[0] & kBadCount) return L3_ERR_COUNT;
    if (hdr[0] != 0) return L3_ERR_STATE;
    const int S = hdr[1];
    const int64_t* src = h + 2;
    int64_t* staged = h + 2 + B;
    int64_t total = 0;
    for (int g = 0; g < S; ++g) {
      staged[g] = total;
      total += n_host[g];
    }
    if (total > stage_rows) return L3_ERR_WORKSPACE;
    const int64_t es = static_cast<int64_t>(elem_bytes(d.dtype));
    const int64_t kb = d.d * es, vb = d.d_e * es;
    // one DMA copy per run of ids whose rows are adjacent in the table
    for (int g = 0; g < S && e == hipSuccess;) {
      int g1 = g + 1;
      while (g1 < S && src[g1] == src[g1 - 1] + n_host[g1 - 1]) ++g1;
      const int64_t rows = staged[g1 - 1] + n_host[g1 - 1] - staged[g];
      e = hipMemcpyAsync(static_cast<uint8_t*>(K_stage) + staged[g] * kb,
                         static_cast<const uint8_t*>(K_host) + src[g] * kb,
                         rows * kb, hipMemcpyHostToDevice, s);
      if (e == hipSuccess)
        e = hipMemcpyAsync(static_cast<uint8_t*>(V_stage) + staged[g] * vb,
                           static_cast<const uint8_t*>(V_host) + src[g] * vb,
                           rows * vb, hipMemcpyHostToDevice, s);
      g = g1;
    }
    // the plan's row offsets now point into the staged tables (a kernel
    // reading the pinned mirror: no memset or copy node in the stream)
    if (e == hipSuccess) {
      const void* staged_dev = nullptr;
      if (!device_readable(staged, &staged_dev)) return L3_ERR_HIP;
      copy_i64_kernel<<<(S + 255) / 256, 256, 0, s>>>(
          pd.seg_row_off, static_cast<const int64_t*>(staged_dev), S);
      e = hipGetLastError();
    }
    if (e != hipSuccess) return L3_ERR_HIP;
    plan->staged = true;
    plan->saved.clear();
    return finish(plan, e, s);
  } catch (...) {
    return L3_ERR_HIP;
  }
}

l3_status l3_plan_info(l3_plan_t plan, int64_t* info, int n, void* stream) {
  if (!plan || (!info && n > 0)) return L3_ERR_NULL;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess)
    return L3_ERR_HIP;
  int32_t hdr[4] = {0, 0, 0, 0};
  if (plan->B > 0 && hipMemcpy(hdr, plan->dev.header, sizeof(hdr),
                               hipMemcpyDeviceToHost) != hipSuccess)
    return L3_ERR_HIP;
  const int64_t v[6] = {plan->B, hdr[1], hdr[2], hdr[3], plan->chunk_rows,
                        plan->group_min_rows};
  for (int i = 0; i < n && i < 6; ++i) info[i] = v[i];
  return L3_OK;
}

l3_status l3_plan_export(l3_plan_t plan, int32_t* perm, int32_t* S,
                         int32_t* seg_id, int32_t* seg_tok_start,
                         int64_t* seg_row_off, int32_t* seg_n, void* stream) {
  if (!plan) return L3_ERR_NULL;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess)
    return L3_ERR_HIP;
  const int64_t B = plan->B;
  int32_t hdr[4] = {0, 0, 0, 0};
  if (B > 0 && hipMemcpy(hdr, plan->dev.header, sizeof(hdr),
                         hipMemcpyDeviceToHost) != hipSuccess)
    return L3_ERR_HIP;
  const int64_t nS = hdr[1];
  if (S) *S = static_cast<int32_t>(nS);
  auto cp = [](void* dst, const void* src, size_t bytes) {
    return bytes == 0 || !dst ||
           hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost) == hipSuccess;
  };
  bool ok = true;
  if (B > 0) {
    ok = ok && cp(perm, plan->dev.perm, B * sizeof(int32_t));
    ok = ok && cp(seg_id, plan->dev.seg_id, nS * sizeof(int32_t));
    ok = ok && cp(seg_tok_start, plan->dev.seg_tok_start,
                  (nS + 1) * sizeof(int32_t));
    ok = ok && cp(seg_row_off, plan->dev.seg_row_off, nS * sizeof(int64_t));
    ok = ok && cp(seg_n, plan->dev.seg_n, nS * sizeof(int32_t));
  } else if (seg_tok_start) {
    seg_tok_start[0] = 0;
  }
  return ok ? L3_OK : L3_ERR_HIP;
}

l3_status l3_forward(l3_plan_t plan, const void* x, const void* K,
                     const void* V, const void* W_up, const void* gamma,
                     const void* beta, const void* W_mix, void* y, void* save,
                     size_t save_bytes, void* scratch_ws, size_t scratch_bytes,
                     void* stream) {
  try {
    if (!plan) return L3_ERR_NULL;
    const int64_t B = plan->B;
    if (B == 0) return L3_OK;
    if (!x || !K || !V || !W_up || !gamma || !beta || !W_mix || !y ||
        !scratch_ws)
      return L3_ERR_NULL;
    const l3_desc& d = plan->desc;
    if (scratch_bytes < fwd_bytes_for(d, B) || !aligned(scratch_ws))
      return L3_ERR_WORKSPACE;
    if (save && (save_bytes < save_bytes_for(d, B) || !aligned(save)))
      return L3_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Carver cs(scratch_ws);
    FwdBufs f = carve_fwd(cs, d, B);
    SaveBufs sv{nullptr, nullptr, nullptr, nullptr};
    if (save) {
      Carver cv(save);
      sv = carve_save(cv, d, B);
    }
    const PlanDev& pd = plan->dev;
    hipError_t e = hipSuccess;

    SegFwdArgs sa;
    sa.header = pd.header;
    sa.perm = pd.perm;
    sa.seg_tok_start = pd.seg_tok_start;
    sa.seg_row_off = pd.seg_row_off;
    sa.seg_n = pd.seg_n;
    // Training runs every id through the wave kernel, whose weights then
    // stay float32 (the group kernel multiplies bf16 weights on MFMA, too
    // coarse for the saved aggregate the gradients are built from).
    const bool all_wave = save != nullptr && plan->group_min_rows > 0;
    sa.seg_item_start = all_wave ? pd.seg_aitem_start : pd.seg_item_start;
    sa.item_map = all_wave ? pd.aitem_map : pd.item_map;
    sa.count_slot = all_wave ? 8 : 2;
    sa.x = x;
    sa.K = K;
    sa.V = V;
    sa.d = d.d;
    sa.d_e = d.d_e;
    sa.chunk_rows = plan->chunk_rows;
    sa.nch_max = plan->nch_max;
    sa.a_out = f.a_act;
    sa.a_save = sv.a32;
    sa.part = f.part;
    sa.part_ml = f.part_ml;
    const int64_t distinct = B < d.vocab ? B : d.vocab;
    const int64_t items_ub = ((B + kTokTile - 1) / kTokTile + distinct) *
                             static_cast<int64_t>(plan->nch_max);
    // With the group kernel enabled (inference), one launch of it runs every
    // item: the busy ids' 128-token items, the 64-token items and the wave
    // items (one per wavefront), all from device-wide queues, so no
    // workgroup idles while another still has work.
    const bool merged = plan->group_min_rows > 0 && !all_wave;
    if (!merged) {
      StageTimer t(plan, ST_SEG, s);
      e = seg_fwd_launch(sa, d.dtype, static_cast<int>(B),
                         static_cast<int>(items_ub < (1 << 30) ? items_ub
                                                               : (1 << 30)),
                         s);
    } else {
      SegGroupArgs ga;
      ga.header = pd.header;
      ga.perm = pd.perm;
      ga.seg_tok_start = pd.seg_tok_start;
      ga.seg_row_off = pd.seg_row_off;
      ga.seg_n = pd.seg_n;
      ga.seg_gitem_start = pd.seg_gitem_start;
      ga.gitem_map = pd.gitem_map;
      ga.hitem_map = pd.hitem_map;
      ga.hcap = static_cast<int>(hitem_cap(B));
      ga.work = pd.header + 4;
      ga.x = static_cast<const uint16_t*>(x);
      ga.K = static_cast<const uint16_t*>(K);
      ga.V = static_cast<const uint16_t*>(V);
      ga.d = d.d;
      ga.d_e = d.d_e;
      ga.a_out = static_cast<uint16_t*>(f.a_act);
      ga.a_save = sv.a32;
      ga.wave = sa;
      const int64_t gitems_ub =
          (B + kGroupTok - 1) / kGroupTok + distinct + items_ub;
      StageTimer t(plan, ST_GROUP, s);
      e = seg_group_launch(
          ga, static_cast<int>(gitems_ub < (1 << 30) ? gitems_ub : (1 << 30)),
          s);
    }
    if (e != hipSuccess) return L3_ERR_HIP;
    // Row chunks exist only for ids with more rows than one wave item takes;
    // when all such ids go to the group kernel nothing needs merging.
    const bool split =
        plan->nch_max > 1 &&
        (all_wave || !(plan->group_min_rows > 0 &&
                       plan->group_min_rows <= plan->chunk_rows));
    if (split) {
      CombineArgs ca;
      ca.group_min_rows = all_wave ? 0 : plan->group_min_rows;
      ca.header = pd.header;
      ca.perm = pd.perm;
      ca.seg_tok_start = pd.seg_tok_start;
      ca.seg_n = pd.seg_n;
      ca.B = static_cast<int>(B);
      ca.d_e = d.d_e;
      ca.chunk_rows = plan->chunk_rows;
      ca.nch_max = plan->nch_max;
      ca.part = f.part;
      ca.part_ml = f.part_ml;
      ca.a_out = f.a_act;
      ca.a_save = sv.a32;
      StageTimer t(plan, ST_COMBINE, s);
      e = seg_combine_launch(ca, d.dtype, s);
      if (e != hipSuccess) return L3_ERR_HIP;
    }
    // u = a W_up^T  (float32 out). When training, the float32 aggregate is
    // the operand, so the saved LayerNorm state carries no bf16 rounding of a.
    GemmArgs up{};
    up.A1 = save ? static_cast<const void*>(sv.a32) : f.a_act;
    up.A2 = up.A1;
    up.a1_m = up.a2_m = d.d_e;
    up.a1_k = up.a2_k = 1;
    up.K1 = d.d_e;
    up.Bm = W_up;
    up.b_k = 1;
    up.b_n = d.d_e;
    up.C = f.U;
    up.c_m = d.d;
    up.M = static_cast<int>(B);
    up.N = d.d;
    up.K = d.d_e;
    up.header = pd.header;
    // y = [h ; x] W_mix^T, the A operand switching from h to x at k = d
    GemmArgs mx{};
    mx.A1 = f.h_act;
    mx.A2 = x;
    mx.a1_m = mx.a2_m = d.d;
    mx.a1_k = mx.a2_k = 1;
    mx.K1 = d.d;
    mx.Bm = W_mix;
    mx.b_k = 1;
    mx.b_n = 2 * static_cast<int64_t>(d.d);
    mx.C = y;
    mx.c_m = d.d;
    mx.M = static_cast<int>(B);
    mx.N = d.d;
    mx.K = 2 * d.d;
    mx.header = pd.header;
    // Inference on bf16 with an MFMA GEMM. With both projections on 256 x
    // 256 tiles, LayerNorm is folded into W_mix: u is written as bf16, the
    // W_up epilogue writes per-row partial statistics, gamma and beta are
    // folded into a bf16 copy of W_mix's first d columns, and W_mix reads u
    // itself (h is never written). Otherwise (small batches) u is written
    // in float32 and the row kernel normalises it, as for training (no
    // centred copy of W_up is needed: float32 u keeps its spread through
    // the mean's cancellation); training and float32 keep u in float32
    // for the saved state.
    const bool mfma_up = !save && d.dtype == L3_BF16 && gemm_nt_mfma_ok(up);
    const int64_t fold_w1 = static_cast<int64_t>(d.d) * d.d * 2;
    const int64_t fold_c = static_cast<int64_t>(d.d) * 8;
    const int64_t fold_st = B * (d.d / 256) * 8;
    const int64_t fold_rows = B * 8;
    const bool fold_ok = mfma_up && !f.gpart && d.d % 256 == 0 &&
                         gemm_nt_256_ok(up) && gemm_nt_256_ok(mx) &&
                         fold_w1 + fold_c + fold_st + fold_rows <= B * d.d * 2;
    // Large batches go one step further: W_up itself is folded through
    // LayerNorm into W_mix, so u is never formed. With Wc = W_up with its
    // columns centred over the d outputs, u - mean(u) = Wc a, hence
    //   var(u) = a^T G a / d,  G = Wc^T Wc            (d_e x d_e)
    //   W_mix1 h = rstd * (Mc a) + W_mix1 beta,  Mc = W_mix1 diag(gamma) Wc
    // (d x d_e). G and Mc are products of the weights (per call, hi | lo
    // operands on the bf16 kernel); per row, a^T G a comes from a GEMM
    // a G whose epilogue dots each row with a itself, and y takes
    // [a ; x] against [Mc | W_mix2] over K = d_e + d instead of 2d.
    const int64_t DD = d.d, DE = d.d_e;
    auto al = [](int64_t v) { return (v + 255) & ~int64_t(255); };
    const int64_t o_t = al(4 * DD * DD), o_mt = al(o_t + 6 * DE * DD),
                  o_g = al(o_mt + 2 * DD * DE), o_gh = al(o_g + 4 * DE * DE),
                  o_gl = al(o_gh + 2 * DE * DE), o_mean = al(o_gl + 2 * DE * DE),
                  o_part = al(o_mean + 4 * DE * ((DD + 63) / 64));
    const int64_t q_c = al(DD * 8), q_st = al(B * (DE / 256) * 8);
    const bool fuse_up = fold_ok && DE % 256 == 0 && fuse_up_pays(B, DD, DE) &&
                         o_part + (int64_t(16) << 20) <= B * DD * 4 &&
                         q_c + q_st + B * 8 <= B * DD * 2;
    const bool fold = fold_ok && !fuse_up;
    // bf16 u only where it feeds the LayerNorm fold
    const bool u_bf16 = fold;
    // Where u is stored as bf16, it is formed from W_up with its columns
    // centred over the d outputs (as bf16 hi | lo over K = 2 d_e, the
    // aggregate read for both halves): u - mean(u) = Wc a exactly, and
    // LayerNorm's output does not change when its input is shifted by the
    // row's mean, so u's rounding is relative to its spread rather than to
    // a mean that may be many times larger.
    if (u_bf16 && !fuse_up) {
      {
        StageTimer t(plan, ST_UP, s);
        e = center_split_launch(pd.header, static_cast<const uint16_t*>(W_up),
                                d.d, d.d_e, f.wc_part, f.wc, s);
      }
      if (e != hipSuccess) return L3_ERR_HIP;
      up.Bm = f.wc;
      up.b_n = 2 * static_cast<int64_t>(d.d_e);
      up.K = 2 * d.d_e;
    }
    LnRowsArgs lr{};
    if (fuse_up) {
      char* ub = reinterpret_cast<char*>(f.U);
      char* hb = static_cast<char*>(f.h_act);
      float* part = reinterpret_cast<float*>(ub + o_part);
      const int64_t part_floats = (B * DD * 4 - o_part) / 4;
      uint16_t* w1s = reinterpret_cast<uint16_t*>(ub);
      uint16_t* tw = reinterpret_cast<uint16_t*>(ub + o_t);
      uint16_t* mt = reinterpret_cast<uint16_t*>(ub + o_mt);
      float* gm = reinterpret_cast<float*>(ub + o_g);
      uint16_t* gh = reinterpret_cast<uint16_t*>(ub + o_gh);
      uint16_t* gl = reinterpret_cast<uint16_t*>(ub + o_gl);
      float* c12 = reinterpret_cast<float*>(hb);
      float* stats = reinterpret_cast<float*>(hb + q_c);
      float* rows = reinterpret_cast<float*>(hb + q_c + q_st);
      {
        StageTimer t(plan, ST_WFOLD, s);
        // c12 = (0, W_mix1 beta); W_mix1 diag(gamma) itself is not formed
        LnFoldArgs fa;
        fa.header = pd.header;
        fa.W = static_cast<const uint16_t*>(W_mix);
        fa.w_n = 2 * DD;
        fa.gamma = static_cast<const uint16_t*>(gamma);
        fa.beta = static_cast<const uint16_t*>(beta);
        fa.n = d.d;
        fa.d = d.d;
        fa.W1 = nullptr;
        fa.c12 = c12;
        fa.split = 1;
        // Wc^T as [hi | hi | lo] (d_e x 3d) and (diag(gamma) Wc)^T as
        // [hi | lo] (d_e x 2d, in the first buffer); c12 and Wc's column
        // sums share one launch
        e = fold_prep_launch(fa, static_cast<const uint16_t*>(W_up), d.d,
                             d.d_e, reinterpret_cast<float*>(ub + o_mean), tw,
                             static_cast<const uint16_t*>(gamma), w1s, s);
        // Mc = [W_mix1 | W_mix1] . [(gamma Wc) hi | lo] over K = 2d (bf16:
        // W_mix1 is exact); up to 8 K shares here and 16 for G (more shares
        // made the in-order sum of the partials cost more than the GEMM
        // saved)
        GemmArgs gw{};
        gw.A1 = W_mix;
        gw.A2 = W_mix;
        gw.a1_m = gw.a2_m = 2 * DD;
        gw.a1_k = gw.a2_k = 1;
        gw.K1 = d.d;
        gw.Bm = w1s;
        gw.b_k = 1;
        gw.b_n = 2 * DD;
        gw.C = mt;
        gw.c_m = DE;
        gw.M = d.d;
        gw.N = d.d_e;
        gw.K = 2 * d.d;
        gw.header = pd.header;
        // G = [hi | lo | hi] . [hi | hi | lo] of Wc^T (float32 sums, then
        // hi | lo), side by side with Mc in one launch where they fit
        GemmArgs gg = gw;
        gg.A1 = tw + DD;
        gg.A2 = tw;
        gg.a1_m = gg.a2_m = 3 * DD;
        gg.K1 = 2 * d.d;
        gg.Bm = tw;
        gg.b_n = 3 * DD;
        gg.K = 3 * d.d;
        gg.C = gm;
        gg.M = d.d_e;
        GemmArgs gp = gg;
        gp.C = gh;
        gp.c_m = DE;
        hipError_t pe = hipErrorInvalidValue;
        if (e == hipSuccess)
          pe = gemm_nt_256_splitk_pair_launch(gw, 8, gp, 16, gl, part,
                                              part_floats, s);
        if (e == hipSuccess && pe != hipSuccess) {
          if (pe != hipErrorInvalidValue) return L3_ERR_HIP;
          e = gemm_nt_256_splitk_launch(gw, s, part, part_floats, 8, kBF16);
          if (e == hipSuccess)
            e = gemm_nt_256_splitk_launch(gg, s, part, part_floats, 16, kF32);
          if (e == hipSuccess)
            e = split_bf16_launch(pd.header, gm, DE * DE, gh, gl, s);
        }
        if (e != hipSuccess) return L3_ERR_HIP;
      }
      // per row a^T G a: a (G_hi + G_lo), each row dotted with a
      GemmArgs gq{};
      gq.A1 = f.a_act;
      gq.A2 = f.a_act;
      gq.a1_m = gq.a2_m = DE;
      gq.a1_k = gq.a2_k = 1;
      gq.K1 = d.d_e;
      gq.B1 = gh;
      gq.b1_n = DE;
      gq.Bm = gl;
      gq.b_k = 1;
      gq.b_n = DE;
      gq.b2_rel = 1;
      gq.M = static_cast<int>(B);
      gq.N = d.d_e;
      gq.K = 2 * d.d_e;
      gq.header = pd.header;
      gq.ln_stats_out = stats;
      gq.ln_quad_a = static_cast<const uint16_t*>(f.a_act);
      gq.ln_quad_lda = DE;
      {
        StageTimer t(plan, ST_UP_QUAD, s);
        e = gemm_nt_256_quad_launch(gq, s);
      }
      if (e != hipSuccess) return L3_ERR_HIP;
      lr.header = pd.header;
      lr.part = stats;
      lr.nparts = d.d_e / 256;
      lr.B = static_cast<int>(B);
      lr.d = d.d;
      lr.eps = d.ln_eps;
      lr.rows = rows;
      lr.quad = 1;
      {
        StageTimer t(plan, ST_LN, s);
        e = ln_rows_launch(lr, s);
      }
      if (e != hipSuccess) return L3_ERR_HIP;
      mx.A1 = f.a_act;
      mx.a1_m = DE;
      mx.K1 = d.d_e;
      mx.B1 = mt;
      mx.b1_n = DE;
      mx.Bm = static_cast<const uint16_t*>(W_mix) + DD;
      mx.b2_rel = 1;
      mx.K = d.d_e + d.d;
      mx.ln_rows = rows;
      mx.ln_c12 = c12;
    }
    if (fold) {
      char* base = static_cast<char*>(f.h_act);
      LnFoldArgs fa;
      fa.header = pd.header;
      fa.W = static_cast<const uint16_t*>(W_mix);
      fa.w_n = 2 * static_cast<int64_t>(d.d);
      fa.gamma = static_cast<const uint16_t*>(gamma);
      fa.beta = static_cast<const uint16_t*>(beta);
      fa.n = d.d;
      fa.d = d.d;
      fa.W1 = reinterpret_cast<uint16_t*>(base);
      fa.c12 = reinterpret_cast<float*>(base + fold_w1);
      float* stats = reinterpret_cast<float*>(base + fold_w1 + fold_c);
      float* rows = reinterpret_cast<float*>(base + fold_w1 + fold_c + fold_st);
      up.ln_stats_out = stats;
      lr.header = pd.header;
      lr.part = stats;
      lr.nparts = d.d / 256;
      lr.B = static_cast<int>(B);
      lr.d = d.d;
      lr.eps = d.ln_eps;
      lr.rows = rows;
      mx.A1 = f.U;
      mx.B1 = fa.W1;
      mx.b1_n = d.d;
      mx.ln_rows = rows;
      mx.ln_c12 = fa.c12;
      StageTimer t(plan, ST_LN, s);
      e = ln_fold_launch(fa, s);
      if (e != hipSuccess) return L3_ERR_HIP;
    }
    // Training on bf16: the float32 aggregate enters as bf16 hi | lo halves
    // over a doubled K, W_up read for both halves (a_hi W_up^T + a_lo
    // W_up^T in one reduction) on the 256 x 256 bf16 kernel.
    GemmArgs u2 = up;
    u2.A1 = f.a_hi;
    u2.A2 = f.a_lo;
    u2.B1 = W_up;
    u2.b1_n = d.d_e;
    u2.b2_rel = 1;
    u2.K = 2 * d.d_e;
    const bool u_split = save && f.a_hi && gemm_nt_256_ok(u2);
    LnArgs ln;
    ln.header = pd.header;
    ln.U = f.U;
    ln.gamma = gamma;
    ln.beta = beta;
    ln.B = static_cast<int>(B);
    ln.d = d.d;
    ln.eps = d.ln_eps;
    ln.h = f.h_act;
    ln.h_save = sv.h32;
    ln.uhat_save = sv.uhat;
    ln.rstd_save = sv.rstd;
    if (!fuse_up) {  // (else u is not formed)
      StageTimer t(plan, ST_UP, s);
      if (u_bf16) {
        e = gemm_nt_mfma_launch(up, kBF16, s, f.gpart, f.gpart_floats);
      } else if (mfma_up) {
        // float32 u and its LayerNorm (at few rows one kernel sums the K
        // shares and normalises)
        e = gemm_ln_launch(up, ln, d.dtype, s, f.gpart, f.gpart_floats);
      } else if (u_split) {
        e = split_bf16_launch(pd.header, sv.a32, B * d.d_e, f.a_hi, f.a_lo,
                              s);
        if (e == hipSuccess)
          e = gemm_nt_256_splitk_launch(u2, s, nullptr, 0);
      } else {
        e = gemm_launch(up, save ? kF32 : d.dtype, d.dtype, kF32, s);
      }
    }
    if (e != hipSuccess) return L3_ERR_HIP;
    if (fold) {
      StageTimer t(plan, ST_LN, s);
      e = ln_rows_launch(lr, s);
    }
    if (e != hipSuccess) return L3_ERR_HIP;
    // (with the W_up fold u is not formed; float32 inference u was
    // normalised with its product)
    if (!u_bf16 && !fuse_up && !mfma_up) {
      StageTimer t(plan, ST_LN, s);
      e = ln_launch(ln, d.dtype, s);
    }
    if (e != hipSuccess) return L3_ERR_HIP;
    {
      StageTimer t(plan, fuse_up ? ST_MIX_UP : ST_MIX, s);
      if (d.dtype == L3_BF16 && gemm_nt_mfma_ok(mx))
        e = gemm_nt_mfma_launch(mx, d.y_dtype, s, f.gpart, f.gpart_floats);
      else
        e = gemm_launch(mx, d.dtype, d.dtype, d.y_dtype, s);
    }
    l3_status st = finish(plan, e, s);
    if (st == L3_OK && save) {
      bool known = false;
      for (const void* p : plan->saved) known = known || p == save;
      if (!known) {
        if (plan->saved.size() >= 1024) plan->saved.erase(plan->saved.begin());
        plan->saved.push_back(save);
      }
    }
    return st;
  } catch (...) {
    return L3_ERR_HIP;
  }
}

l3_status l3_backward(l3_plan_t plan, const void* dy, const void* x,
                      const void* K, const void* V, const void* W_up,
                      const void* gamma, const void* beta, const void* W_mix,
                      const void* save, size_t save_bytes, float* dx,
                      float* dK, float* dV, float* dW_up, float* dgamma,
                      float* dbeta, float* dW_mix, void* scratch_ws,
                      size_t scratch_bytes, void* stream) {
  try {
    if (!plan) return L3_ERR_NULL;
    const l3_desc& d = plan->desc;
    const int64_t B = plan->B;
    if (!dK || !dV || !dW_up || !dgamma || !dbeta || !dW_mix) return L3_ERR_NULL;
    if (B > 0 && (!dy || !x || !K || !V || !W_up || !gamma || !beta ||
                  !W_mix || !save || !dx || !scratch_ws))
      return L3_ERR_NULL;
    (void)beta;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    const int64_t es = static_cast<int64_t>(elem_bytes(d.dtype));
    if (B == 0) {
      // no tokens: every gradient is zero
      e = fill_zero_launch(dK, d.rows * d.d, s);
      if (e == hipSuccess) e = fill_zero_launch(dV, d.rows * d.d_e, s);
      if (e == hipSuccess) e = fill_zero_launch(dW_up, int64_t(d.d) * d.d_e, s);
      if (e == hipSuccess) e = fill_zero_launch(dgamma, d.d, s);
      if (e == hipSuccess) e = fill_zero_launch(dbeta, d.d, s);
      if (e == hipSuccess) e = fill_zero_launch(dW_mix, int64_t(d.d) * 2 * d.d, s);
      return finish(plan, e, s);
    }
    bool known = false;
    for (const void* p : plan->saved) known = known || p == save;
    if (!known || plan->staged) return L3_ERR_STATE;
    if (save_bytes < save_bytes_for(d, B) || !aligned(save))
      return L3_ERR_WORKSPACE;
    if (scratch_bytes < bwd_bytes_for(d, B) || !aligned(scratch_ws))
      return L3_ERR_WORKSPACE;
    Carver cv(const_cast<void*>(save));
    SaveBufs sv = carve_save(cv, d, B);
    Carver cs(scratch_ws);
    BwdBufs bb = carve_bwd(cs, d, B);
    const PlanDev& pd = plan->dev;
    const int Bi = static_cast<int>(B);
    const int64_t D = d.d, DE = d.d_e;
    {
      StageTimer t(plan, ST_BWD_MIX, s);
      // dH = dY W_a, dx = dY W_b (W_a = W_mix[:, :d], W_b = W_mix[:, d:]).
      // bf16: both operands are bf16 inputs, so bf16 MFMA with float32
      // accumulation forms the same exact products as float32 arithmetic;
      // it needs W_mix transposed (the reduction index j last).
      GemmArgs t16{};
      t16.A1 = t16.A2 = dy;
      t16.a1_m = t16.a2_m = D;
      t16.a1_k = t16.a2_k = 1;
      t16.K1 = d.d;
      t16.Bm = bb.wmixT;
      t16.b_k = 1;
      t16.b_n = D;
      t16.C = bb.dH;
      t16.c_m = D;
      t16.M = Bi;
      t16.N = d.d;
      t16.K = d.d;
      t16.header = pd.header;
      const bool mfma = bb.wmixT && gemm_nt_mfma_ok(t16);
      if (mfma) {
        e = transpose_bf16_launch(pd.header,
                                  static_cast<const uint16_t*>(W_mix), 2 * D,
                                  d.d, 2 * d.d, bb.wmixT, s);
        if (e == hipSuccess) e = gemm_nt_mfma_launch(t16, kF32, s);
        if (e == hipSuccess) {
          t16.Bm = bb.wmixT + D * D;
          t16.C = dx;
          e = gemm_nt_mfma_launch(t16, kF32, s);
        }
      }
      // otherwise B(k=j, n) = W_mix[j, n] read in place (generic kernel)
      GemmArgs g{};
      g.A1 = g.A2 = dy;
      g.a1_m = g.a2_m = D;
      g.a1_k = g.a2_k = 1;
      g.K1 = d.d;
      g.Bm = W_mix;
      g.b_k = 2 * D;
      g.b_n = 1;
      g.C = bb.dH;
      g.c_m = D;
      g.M = Bi;
      g.N = d.d;
      g.K = d.d;
      g.header = pd.header;
      if (!mfma) {
        e = gemm_launch(g, d.dtype, d.dtype, kF32, s);
        if (e == hipSuccess) {
          g.Bm = static_cast<const char*>(W_mix) + D * es;
          g.C = dx;
          e = gemm_launch(g, d.dtype, d.dtype, kF32, s);
        }
      }
      // dW_mix[:, :d] = dY^T H, dW_mix[:, d:] = dY^T X  (sums over tokens).
      // bf16: on the 256 x 256 bf16 kernel with K split, from transposed
      // copies (tokens last): dY^T X has bf16 operands (exact products);
      // the float32 H enters as hi + lo bf16 halves over a doubled K
      // (dY^T repeated), i.e. dY^T H_hi + dY^T H_lo in one reduction.
      bool wmfma = false;
      GemmArgs wx{};
      if (e == hipSuccess && bb.dyT) {
        wx.A1 = wx.A2 = bb.dyT;
        wx.a1_m = wx.a2_m = B;
        wx.a1_k = wx.a2_k = 1;
        wx.K1 = Bi;
        wx.Bm = bb.xT;
        wx.b_k = 1;
        wx.b_n = B;
        wx.C = dW_mix + D;
        wx.c_m = 2 * D;
        wx.M = d.d;
        wx.N = d.d;
        wx.K = Bi;
        wx.header = pd.header;
        GemmArgs wh = wx;
        wh.Bm = bb.hT;
        wh.b_n = 2 * B;
        wh.K = 2 * Bi;
        wh.C = dW_mix;
        wmfma = gemm_nt_256_ok(wx) && gemm_nt_256_ok(wh);
        if (wmfma) {
          e = transpose_bf16_launch(pd.header,
                                    static_cast<const uint16_t*>(dy), D, Bi,
                                    d.d, bb.dyT, s);
          if (e == hipSuccess)
            e = transpose_bf16_launch(pd.header,
                                      static_cast<const uint16_t*>(x), D, Bi,
                                      d.d, bb.xT, s);
          if (e == hipSuccess)
            e = transpose_split_launch(pd.header, sv.h32, D, Bi, d.d, bb.hT,
                                       s);
          if (e == hipSuccess)
            e = gemm_nt_256_splitk_launch(wh, s, bb.gpart, bb.gpart_floats);
          if (e == hipSuccess)
            e = gemm_nt_256_splitk_launch(wx, s, bb.gpart, bb.gpart_floats);
        }
      }
      if (e == hipSuccess && !wmfma) {
        GemmArgs w{};
        w.A1 = w.A2 = dy;
        w.a1_m = w.a2_m = 1;
        w.a1_k = w.a2_k = D;
        w.K1 = Bi;
        w.Bm = sv.h32;
        w.b_k = D;
        w.b_n = 1;
        w.C = dW_mix;
        w.c_m = 2 * D;
        w.M = d.d;
        w.N = d.d;
        w.K = Bi;
        w.header = pd.header;
        e = gemm_launch(w, d.dtype, kF32, kF32, s, bb.gpart, bb.gpart_floats);
        if (e == hipSuccess) {
          w.Bm = x;
          w.C = dW_mix + D;
          e = gemm_launch(w, d.dtype, d.dtype, kF32, s, bb.gpart,
                          bb.gpart_floats);
        }
      }
    }
    if (e != hipSuccess) return L3_ERR_HIP;
    BwdArgs ba;
    ba.header = pd.header;
    ba.perm = pd.perm;
    ba.seg_tok_start = pd.seg_tok_start;
    ba.seg_row_off = pd.seg_row_off;
    ba.seg_n = pd.seg_n;
    ba.B = Bi;
    ba.d = d.d;
    ba.d_e = d.d_e;
    ba.x = x;
    ba.K = K;
    ba.V = V;
    ba.gamma = gamma;
    ba.uhat = sv.uhat;
    ba.rstd = sv.rstd;
    ba.dH = bb.dH;
    ba.dU = bb.dU;
    ba.dA = bb.dA;
    ba.dx = dx;
    ba.dK = dK;
    ba.dV = dV;
    ba.dgamma = dgamma;
    ba.dbeta = dbeta;
    ba.rows = d.rows;
    // the work items of the saving forward: every id's wave items
    ba.item_map = plan->group_min_rows > 0 ? pd.aitem_map : pd.item_map;
    ba.count_slot = plan->group_min_rows > 0 ? 8 : 2;
    ba.chunk_rows = plan->chunk_rows;
    ba.kst = bwd_kst(d);
    ba.Pbuf = bb.P;
    ba.DSbuf = bb.dS;
    ba.ln_part = bb.ln_part;
    ba.rows_map = bb.rows_map;
    ba.rows_count = bb.rows_count;
    ba.zero_map = bb.zero_map;
    ba.zero_count = bb.zero_count;
    ba.chunk_stats = bb.chunk_stats;
    ba.cs_stride = (d.k_max + 31) / 32;
    ba.gitem_map = plan->group_min_rows > 0 ? pd.gitem_map : nullptr;
    ba.group_min_rows = plan->group_min_rows;
    {
      StageTimer t(plan, ST_BWD_LN, s);
      e = ln_bwd_launch(ba, d.dtype, s);
    }
    if (e != hipSuccess) return L3_ERR_HIP;
    {
      StageTimer t(plan, ST_BWD_UP, s);
      // dW_up = dU^T A (sum over tokens). bf16: both are float32, so three
      // bf16 products hi hi + lo hi + hi lo over K = 3B (the lo lo term is
      // below float32 rounding): A = [dU_hi^T | dU_lo^T] (the h^T buffer,
      // free by now; for k >= 2B the second operand pointer wraps to the
      // hi half), B = [A_hi^T | A_hi^T | A_lo^T] (the dY^T buffer), split K.
      bool wumfma = false;
      if (bb.hT && 3 * d.d_e <= d.d) {
        GemmArgs h{};
        h.A1 = h.A2 = bb.hT;
        h.a1_m = h.a2_m = 2 * B;
        h.a1_k = h.a2_k = 1;
        h.K1 = 2 * Bi;
        h.Bm = bb.dyT;
        h.b_k = 1;
        h.b_n = 3 * B;
        h.C = dW_up;
        h.c_m = DE;
        h.M = d.d;
        h.N = d.d_e;
        h.K = 3 * Bi;
        h.header = pd.header;
        wumfma = gemm_nt_256_ok(h);
        if (wumfma) {
          e = transpose_split_launch(pd.header, bb.dU, D, Bi, d.d, bb.hT, s);
          if (e == hipSuccess)
            e = transpose_split_launch(pd.header, sv.a32, DE, Bi, d.d_e,
                                       bb.dyT, s, 3 * B, 2 * B, B);
          if (e == hipSuccess)
            e = gemm_nt_256_splitk_launch(h, s, bb.gpart, bb.gpart_floats, 64);
        }
      }
      GemmArgs w{};
      w.A1 = w.A2 = bb.dU;
      w.a1_m = w.a2_m = 1;
      w.a1_k = w.a2_k = D;
      w.K1 = Bi;
      w.Bm = sv.a32;
      w.b_k = DE;
      w.b_n = 1;
      w.C = dW_up;
      w.c_m = DE;
      w.M = d.d;
      w.N = d.d_e;
      w.K = Bi;
      w.header = pd.header;
      if (!wumfma)
        e = gemm_launch(w, kF32, kF32, kF32, s, bb.gpart, bb.gpart_floats);
      // dA = dU W_up. bf16: the float32 dU enters as bf16 hi | lo halves
      // (in the dY^T / x^T buffers, free by now) over a doubled K, against
      // [W_up^T | W_up^T] (in the W_mix^T buffer): dU_hi W_up + dU_lo W_up
      // in one reduction, on the 256 x 256 bf16 kernel.
      bool amfma = false;
      if (e == hipSuccess && bb.dyT && d.d_e <= d.d) {
        GemmArgs h{};
        h.A1 = bb.dyT;
        h.A2 = bb.xT;
        h.a1_m = h.a2_m = D;
        h.a1_k = h.a2_k = 1;
        h.K1 = d.d;
        h.Bm = bb.wmixT;
        h.b_k = 1;
        h.b_n = 2 * D;
        h.C = bb.dA;
        h.c_m = DE;
        h.M = Bi;
        h.N = d.d_e;
        h.K = 2 * d.d;
        h.header = pd.header;
        amfma = gemm_nt_256_ok(h);
        if (amfma) {
          e = split_bf16_launch(pd.header, bb.dU, B * D, bb.dyT, bb.xT, s);
          const uint16_t* wu = static_cast<const uint16_t*>(W_up);
          if (e == hipSuccess)
            e = transpose_bf16_launch(pd.header, wu, DE, d.d, d.d_e, bb.wmixT,
                                      s, 2 * D);
          if (e == hipSuccess)
            e = transpose_bf16_launch(pd.header, wu, DE, d.d, d.d_e,
                                      bb.wmixT + D, s, 2 * D);
          if (e == hipSuccess)
            e = gemm_nt_256_splitk_launch(h, s, bb.gpart, bb.gpart_floats);
        }
      }
      if (e == hipSuccess && !amfma) {
        GemmArgs g{};
        g.A1 = g.A2 = bb.dU;
        g.a1_m = g.a2_m = D;
        g.a1_k = g.a2_k = 1;
        g.K1 = d.d;
        g.Bm = W_up;
        g.b_k = DE;
        g.b_n = 1;
        g.C = bb.dA;
        g.c_m = DE;
        g.M = Bi;
        g.N = d.d_e;
        g.K = d.d;
        g.header = pd.header;
        e = gemm_launch(g, kF32, d.dtype, kF32, s);
      }
    }
    if (e != hipSuccess) return L3_ERR_HIP;
    {
      StageTimer t(plan, ST_BWD_SEG, s);
      // rows of absent ids only (the column pass writes the present ones);
      // float4 stores need d, d_e multiples of 4, row indices int32
      if (D % 4 == 0 && DE % 4 == 0 && d.rows < (int64_t(1) << 31)) {
        e = zero_absent_launch(ba, zero_items_for(d, B), s);
      } else {
        e = fill_zero_launch(dK, d.rows * D, s);
        if (e == hipSuccess) e = fill_zero_launch(dV, d.rows * DE, s);
      }
      const int64_t distinct = B < d.vocab ? B : d.vocab;
      const int64_t items_ub =
          ((B + kTokTile - 1) / kTokTile + distinct) *
          static_cast<int64_t>(plan->nch_max);
      if (e == hipSuccess)
        e = seg_bwd_launch(
            ba, d.dtype,
            static_cast<int>(items_ub < (1 << 30) ? items_ub : (1 << 30)),
            static_cast<int>(distinct), s);
    }
    return finish(plan, e, s);
  } catch (...) {
    return L3_ERR_HIP;
  }
}

l3_status l3_timing_enable(l3_plan_t plan, int enable) {
  if (!plan) return L3_ERR_NULL;
  plan->timing = enable != 0;
  return L3_OK;
}

l3_status l3_timing_read(l3_plan_t plan, double* ms, int64_t* count,
                         int max_stages, int* n_stages) {
  if (!plan) return L3_ERR_NULL;
  if (n_stages) *n_stages = ST_COUNT;
  std::vector<double> acc(ST_COUNT, 0.0);
  std::vector<int64_t> cnt(ST_COUNT, 0);
  l3_status st = L3_OK;
  for (auto& e : plan->events) {
    float v = 0.f;
    if (hipEventSynchronize(e.b) != hipSuccess ||
        hipEventElapsedTime(&v, e.a, e.b) != hipSuccess)
      st = L3_ERR_HIP;
    acc[e.stage] += v;
    cnt[e.stage] += 1;
    hipEventDestroy(e.a);
    hipEventDestroy(e.b);
  }
  plan->events.clear();
  for (int i = 0; i < max_stages && i < ST_COUNT; ++i) {
    if (ms) ms[i] = acc[i];
    if (count) count[i] = cnt[i];
  }
  return st;
}

}  // extern "C"

// ---- allocation-free inference forward -----------------------------------
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops): the forward's scratch workspace is this file-scope device
// array instead of caller memory. Each GPU the library runs on holds its
// own copy, at its own address, until the process ends. In host code the
// array's name is only a host-side stand-in: its device address comes from
// hipGetSymbolAddress, taken once per device with that device current and
// kept below; only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[L3_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (nullptr on a HIP error).
void* static_scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
      return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

l3_status l3_forward_noalloc(l3_plan_t plan, const void* x, const void* K,
                             const void* V, const void* W_up,
                             const void* gamma, const void* beta,
                             const void* W_mix, void* y, void* stream) {
  try {
    if (!plan) return L3_ERR_NULL;
    if (plan->B == 0) return L3_OK;
    // the forward's scratch must fit the static array (checked before any
    // device work, like a caller workspace that is too small)
    if (fwd_bytes_for(plan->desc, plan->B) > L3_NOALLOC_SCRATCH_BYTES)
      return L3_ERR_WORKSPACE;
    void* ptr = static_scratch_ptr();
    if (!ptr) return L3_ERR_HIP;
    // stage timing creates HIP events; this entry point records none
    const bool timing = plan->timing;
    plan->timing = false;
    const l3_status st = l3_forward(plan, x, K, V, W_up, gamma, beta, W_mix,
                                    y, nullptr, 0, ptr,
                                    L3_NOALLOC_SCRATCH_BYTES, stream);
    plan->timing = timing;
    return st;
  } catch (...) {
    return L3_ERR_HIP;
  }
}

}  // extern "C"
