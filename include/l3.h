/*
 * libl3 -- Large Lookup Layer (L3) forward and backward on AMD Instinct
 * MI355X (gfx950). Plain C ABI: host or device pointers, sizes and status
 * codes; no C++ types cross it and no exception escapes it.
 *
 * What is computed (gist.science explainer of "L^3: Large Lookup Layers",
 * Technical Summary, Core Architecture, Mathematical Formulation): for every
 * token i with hidden state x_i and token id t = ids[i],
 *
 *     y_i = W_mix [ LayerNorm( W_up( V_t^T Softmax(K_t x_i) ) ) ; x_i ]
 *
 * where K_t and V_t are the rows offsets[t] .. offsets[t+1]-1 of the key
 * table K [rows x d] and value table V [rows x d_e] (Core Architecture,
 * Static Routing: a pre-computed map from an id to a subset of a large
 * table; Information-Theoretic Embedding Allocation, Constraints: every id
 * owns between 1 and k rows). The batch is first sorted by token id
 * (Systems-Friendly Design, Batch Sorting) so that all tokens of one id
 * share one read of K_t and V_t.
 *
 * Fixed readings of what the pages leave open:
 *   - keys have the width of x (d_k == d); no query projection, no softmax
 *     temperature; W_up [d x d_e] and W_mix [d x 2d] have no bias;
 *   - LayerNorm is over the d features, biased variance, eps = ln_eps,
 *     affine gamma/beta; the concatenation is [LayerNorm output ; x];
 *   - every matrix is row-major and contiguous; weights are [out x in].
 *
 * Memory and streams: the caller owns every buffer. The library never
 * allocates device memory and never synchronises the stream on the plan,
 * forward or backward path (l3_plan_check and l3_plan_export do). All work
 * is queued on the stream passed in (a hipStream_t; NULL is the default
 * stream). Pointers named "device" must be device-accessible; everything
 * else is host memory.
 *
 * Element types: dtype == L3_F32 means every input tensor (x, K, V, W_up,
 * gamma, beta, W_mix, dy) is float32; L3_BF16 means they are bfloat16
 * (uint16 bit patterns). Accumulation is float32 in both cases. y is float32
 * or bfloat16 (y_dtype). Gradients are always float32.
 */
#ifndef L3_H
#define L3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int l3_status;
#define L3_OK 0
#define L3_ERR_NULL (-1)        /* a required pointer is NULL              */
#define L3_ERR_SHAPE (-2)       /* unsupported or inconsistent sizes       */
#define L3_ERR_DTYPE (-3)       /* unknown element type                    */
#define L3_ERR_WORKSPACE (-4)   /* a workspace is smaller than required    */
#define L3_ERR_HIP (-5)         /* a HIP runtime call or launch failed     */
#define L3_ERR_TOKEN_RANGE (-6) /* some id is outside [0, vocab)           */
#define L3_ERR_COUNT (-7)       /* some used id owns 0 or > k_max rows, or
                                   its rows leave [0, rows)                */
#define L3_ERR_STATE (-8)       /* call out of order (e.g. backward without
                                   a forward that saved its activations)  */

#define L3_F32 0
#define L3_BF16 1

/* Largest allowed k_max (the pages' example cap k = 512). */
#define L3_MAX_ROWS_PER_ID 512

typedef struct l3_desc {
  int64_t vocab;   /* V: number of token ids                                 */
  int64_t rows;    /* R: rows of K and V (the offsets' last entry)           */
  int32_t d;       /* hidden width of x and y                                */
  int32_t d_k;     /* key width; must equal d                                */
  int32_t d_e;     /* value width                                            */
  int32_t k_max;   /* largest rows per id, 1 .. L3_MAX_ROWS_PER_ID           */
  int32_t dtype;   /* L3_F32 or L3_BF16, for every input tensor              */
  int32_t y_dtype; /* L3_F32 or L3_BF16                                      */
  float ln_eps;    /* LayerNorm epsilon (1e-5 is the reading used)           */
} l3_desc;

/* Opaque host handle of a plan. It points into the caller's plan workspace
 * and stays valid until l3_plan_release; the workspace must outlive it. */
typedef struct l3_plan_s* l3_plan_t;

/*
 * Sizes: d and d_e must be multiples of 64 and at most 4096, d_k == d,
 * 1 <= k_max <= 512, vocab >= 1, rows >= 1, max_tokens < 2^31.
 *
 * l3_workspace_size: bytes of the three caller-owned device workspaces for
 * batches of up to max_tokens tokens.
 *   plan_ws    -- written by l3_plan, read by l3_forward / l3_backward;
 *   save_ws    -- written by l3_forward when training, read by l3_backward;
 *   scratch_ws -- temporary; its content is never needed between calls.
 * Every workspace must start on a 256-byte boundary (device allocations
 * do); a misaligned one is rejected with L3_ERR_WORKSPACE.
 * Any output pointer may be NULL. Errors: L3_ERR_NULL, L3_ERR_SHAPE,
 * L3_ERR_DTYPE.
 */
l3_status l3_workspace_size(const l3_desc* desc, int64_t max_tokens,
                            size_t* plan_ws, size_t* save_ws,
                            size_t* scratch_ws);

/*
 * l3_plan -- sort a batch by token id and cut it into one segment per id
 * (Systems-Friendly Design, Batch Sorting).
 *   ids      device int32 [B], token ids, each in [0, vocab)
 *   B        number of tokens, 0 <= B <= max_tokens of the workspace
 *   offsets  device int64 [vocab + 1]; id t owns rows offsets[t] ..
 *            offsets[t+1]-1 (Core Architecture, Static Routing)
 *   plan_ws  device workspace of plan_ws_bytes (l3_workspace_size)
 * The sort key is (id, position in the batch), so the permutation and the
 * segments are unique. Host-checkable errors return at once. The id range
 * and the row counts of the ids that occur are checked on the device: a bad
 * value is recorded in the workspace, every later kernel of this plan does
 * nothing, and l3_plan_check reports L3_ERR_TOKEN_RANGE or L3_ERR_COUNT.
 * Only offsets[t], offsets[t+1] of ids t that occur are read.
 * On success *out receives a new handle (free with l3_plan_release).
 * B == 0 is valid: forward and backward then do nothing.
 */
l3_status l3_plan(const l3_desc* desc, const int32_t* ids, int64_t B,
                  const int64_t* offsets, void* plan_ws, size_t plan_ws_bytes,
                  void* stream, l3_plan_t* out);

/*
 * l3_replan -- plan a new batch into an existing handle, reusing its
 * workspace (same rules as l3_plan; B may not exceed the batch size the
 * workspace was sized for). Keeps the handle's timing setting.
 */
l3_status l3_replan(l3_plan_t plan, const int32_t* ids, int64_t B,
                    const int64_t* offsets, void* stream);

/*
 * l3_forward -- y = W_mix [LayerNorm(W_up(V_t^T Softmax(K_t x))) ; x] for
 * the planned batch (Core Architecture, Mathematical Formulation).
 *   x      device [B x d] (dtype)         K      device [rows x d] (dtype)
 *   V      device [rows x d_e] (dtype)    W_up   device [d x d_e] (dtype)
 *   gamma, beta device [d] (dtype)        W_mix  device [d x 2d] (dtype)
 *   y      device [B x d] (y_dtype), overwritten
 *   save   device save workspace (save_bytes), or NULL for inference; when
 *          given, the float32 activations the backward pass needs are kept
 *   scratch device scratch workspace (scratch_bytes)
 * Errors: L3_ERR_NULL, L3_ERR_WORKSPACE, L3_ERR_HIP. Device-detected input
 * errors of the plan make this a no-op (see l3_plan).
 * Inference on bf16 with large batches (when the fold below saves 1e11
 * flops or more: B (2 d d_e + 2 d (d - d_e) - 4 d_e^2) >= 1e11, e.g. 65536
 * tokens at d = 2048, d_e = 512) computes y without forming W_up's output:
 * W_up,
 * with its columns centred, is folded through LayerNorm into W_mix (each
 * row's variance as a quadratic form of the aggregate); the results agree
 * with the unfolded path to bf16 rounding.
 * Forward and backward calls on one plan must not run concurrently (queue
 * them on one stream or synchronise): the plan workspace also holds the
 * forward kernels' work-queue counters, and the scratch workspace is shared.
 */
l3_status l3_forward(l3_plan_t plan, const void* x, const void* K,
                     const void* V, const void* W_up, const void* gamma,
                     const void* beta, const void* W_mix, void* y, void* save,
                     size_t save_bytes, void* scratch, size_t scratch_bytes,
                     void* stream);

/*
 * l3_forward_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the inference forward of l3_forward (save = NULL) with its
 * scratch workspace taken from a static device array of
 * L3_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends. It allocates nothing; the caller still passes
 * the plan, inputs and y (same meaning, layout and ownership as
 * l3_forward). Records no stage timings.
 * Errors: as l3_forward; L3_ERR_WORKSPACE, before any device work, when the
 * planned batch's forward needs more scratch than the array holds (e.g. a
 * 64-token decode batch at d = 2048, d_e = 512 fits; an 8192-token batch at
 * d = 1024 does not); L3_ERR_HIP if the array's device address cannot be
 * obtained. All calls on one GPU share that GPU's array and it keeps the
 * last call's contents: calls that overlap on one GPU (on different
 * streams, or from different host threads without ordering) race and give
 * wrong results; serialise them on one stream.
 */
#define L3_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
l3_status l3_forward_noalloc(l3_plan_t plan, const void* x, const void* K,
                             const void* V, const void* W_up,
                             const void* gamma, const void* beta,
                             const void* W_mix, void* y, void* stream);

/*
 * l3_backward -- gradients of sum(y * dy) for the planned batch, from the
 * state a saving l3_forward on this plan (since its last l3_plan /
 * l3_replan) left in `save` (the pages print no gradients; these are the
 * chain rule of the forward formula). One plan serves every layer that
 * shares the batch's ids and the offsets: each layer calls l3_forward with
 * its own tables, weights and save workspace, and l3_backward with the same.
 *   dy      device [B x d] (dtype)
 *   x, K, V, W_up, gamma, beta, W_mix: the forward's inputs
 *   save    the forward's save workspace (save_bytes)
 *   dx      device float32 [B x d]
 *   dK      device float32 [rows x d]; dV device float32 [rows x d_e]:
 *           every row is written; rows of ids absent from the batch are 0
 *   dW_up   device float32 [d x d_e]; dgamma, dbeta device float32 [d];
 *   dW_mix  device float32 [d x 2d]
 * Every output is overwritten (never accumulated). Every element of dK, dV
 * and every row of dx has one writer, table gradients sum an id's tokens in
 * sorted-batch order, and every other reduction has a fixed order, so
 * results are bitwise reproducible run to run.
 * Errors: L3_ERR_NULL, L3_ERR_WORKSPACE, L3_ERR_HIP, L3_ERR_STATE (`save` was
 * not written by a saving forward on this plan since it was last planned).
 */
l3_status l3_backward(l3_plan_t plan, const void* dy, const void* x,
                      const void* K, const void* V, const void* W_up,
                      const void* gamma, const void* beta, const void* W_mix,
                      const void* save, size_t save_bytes, float* dx,
                      float* dK, float* dV, float* dW_up, float* dgamma,
                      float* dbeta, float* dW_mix, void* scratch,
                      size_t scratch_bytes, void* stream);

/*
 * l3_allocate -- rows per token id (the n_t of the offsets array l3_plan
 * takes) from a budget of embeddings (gist.science explainer,
 * Information-Theoretic Embedding Allocation: an LZW-variant scan of a
 * corpus gives frequent context suffixes more embeddings, every token
 * between 1 and k; Key Contributions: compared with uniform allocation).
 * Host code, run once per model before any batch is planned (LZW's parse
 * is a chain of dependent steps); all pointers are host memory.
 *   method   L3_ALLOC_LZW: the dictionary starts with every single token (one
 *            embedding each); the corpus is parsed as LZW parses it; each
 *            added entry (phrase + next token c) is one more embedding of
 *            c; a token owning k_max embeddings takes no new entry; the
 *            scan stops when the embeddings reach the budget or the corpus
 *            ends (one pass), any budget left unassigned.
 *            L3_ALLOC_UNIFORM: budget / vocab each, the remainder one each
 *            to the lowest ids (the corpus is not read).
 *   corpus   int32 [n_tokens] token ids in [0, vocab) (may be NULL when
 *            n_tokens is 0 or the method is uniform)
 *   vocab    V >= 1; budget in [V, V * k_max]; k_max in [1, 512]
 *   counts   int64 [vocab] out: rows of each id, in [1, k_max]
 *   offsets  int64 [vocab + 1] out (or NULL): exclusive prefix sum of counts
 * Errors: L3_ERR_DTYPE (unknown method), L3_ERR_NULL, L3_ERR_SHAPE,
 * L3_ERR_TOKEN_RANGE (a corpus token outside [0, vocab); nothing written),
 * L3_ERR_WORKSPACE (host memory for the dictionary could not be
 * allocated).
 */
#define L3_ALLOC_UNIFORM 0
#define L3_ALLOC_LZW 1
l3_status l3_allocate(int method, const int32_t* corpus, int64_t n_tokens,
                      int64_t vocab, int64_t budget, int32_t k_max,
                      int64_t* counts, int64_t* offsets);

/*
 * l3_stage_rows -- for tables kept in host memory (gist.science explainer,
 * Systems-Friendly Design: the tables may live in CPU memory because a
 * token's rows follow from its id alone, Core Architecture, Static
 * Routing): copy the rows of every id in the planned batch into compact
 * device tables and point the plan at them. Stream-ordered after the plan;
 * it may run on another stream than the layers before it (order it with an
 * event) so the copy overlaps their work.
 *   K_host   pinned host memory (hipHostMalloc, or a pinned torch
 *            tensor) [rows x d] (dtype), the full key table; device memory
 *            is accepted too; pageable host memory is refused (L3_ERR_NULL)
 *   V_host   the same for the value table [rows x d_e]
 *   K_stage  device [stage_rows x d] (dtype); V_stage device
 *            [stage_rows x d_e]: receive the batch's rows, id by id in
 *            ascending id order
 *   stage_rows capacity in rows; B * k_max always suffices
 * Afterwards l3_forward must be given K_stage, V_stage in place of the full
 * tables, until the next l3_plan / l3_replan of this handle. A staged plan
 * serves inference only: l3_backward returns L3_ERR_STATE, and staging twice
 * without replanning returns L3_ERR_STATE. If the batch's rows exceed
 * stage_rows, nothing is copied, every later kernel of the plan does
 * nothing, and l3_plan_check reports L3_ERR_WORKSPACE.
 * Errors: L3_ERR_NULL, L3_ERR_SHAPE, L3_ERR_STATE, L3_ERR_HIP.
 */
l3_status l3_stage_rows(l3_plan_t plan, const void* K_host,
                        const void* V_host, void* K_stage, void* V_stage,
                        int64_t stage_rows, void* stream);

/*
 * l3_stage_rows_dma -- the same result as l3_stage_rows, with the copies
 * made by the DMA engines (no compute unit is used, so the copy overlaps
 * kernels on other streams): waits for `stream` (which the caller orders
 * after the plan, e.g. with an event, and before nothing else it needs
 * soon), reads the plan's segments to the host, then queues on `stream`
 * one host-to-device copy of K rows and one of V rows per run of ids with
 * adjacent rows, and a small kernel that points the plan at the copies.
 * A pinned host buffer of 32 B per token is allocated with the plan on
 * first use and freed by l3_plan_release; a later call on the plan reuses
 * it, so calls on one plan must not overlap.
 * Errors: as l3_stage_rows, and L3_ERR_WORKSPACE at once (nothing queued)
 * when the rows exceed stage_rows; L3_ERR_TOKEN_RANGE / L3_ERR_COUNT for a
 * plan that failed its device-side checks.
 */
l3_status l3_stage_rows_dma(l3_plan_t plan, const void* K_host,
                            const void* V_host, void* K_stage, void* V_stage,
                            int64_t stage_rows, void* stream);

/*
 * l3_plan_check -- wait for the stream, then report the device-side
 * validation of the plan: L3_OK, L3_ERR_TOKEN_RANGE, L3_ERR_COUNT or
 * L3_ERR_WORKSPACE (staged rows beyond the staging capacity)
 * (L3_ERR_HIP if the stream itself failed).
 */
l3_status l3_plan_check(l3_plan_t plan, void* stream);

/*
 * l3_plan_export -- copy the plan to host memory (waits for the stream).
 *   perm          host int32 [B]    token index at sorted position j
 *   S             host int32 [1]    number of segments (distinct ids)
 *   seg_id        host int32 [B]    first S entries: ids, ascending
 *   seg_tok_start host int32 [B+1]  first S+1 entries: segment starts, then B
 *   seg_row_off   host int64 [B]    first S entries: offsets[id]
 *   seg_n         host int32 [B]    first S entries: rows of the id
 * Any pointer may be NULL to skip that array.
 */
l3_status l3_plan_export(l3_plan_t plan, int32_t* perm, int32_t* S,
                         int32_t* seg_id, int32_t* seg_tok_start,
                         int64_t* seg_row_off, int32_t* seg_n, void* stream);

/*
 * l3_plan_info -- how the forward pass will split the planned batch (waits
 * for the stream). info (host int64) receives up to n of:
 *   [0] B, [1] S (distinct ids), [2] wave-kernel work items,
 *   [3] group-kernel work items, [4] rows per wave-kernel item,
 *   [5] rows from which an id goes to the group kernel (0: group kernel off)
 */
l3_status l3_plan_info(l3_plan_t plan, int64_t* info, int n, void* stream);

/* Free a plan handle (not its workspace). NULL is ignored. */
void l3_plan_release(l3_plan_t plan);

/* Number of tokens of a plan, or -1 for NULL. */
int64_t l3_plan_tokens(l3_plan_t plan);

/* Static description of a status code. */
const char* l3_status_str(l3_status status);

/*
 * Stage timing (measurement aid, off by default). With timing on, every
 * later l3_plan / l3_forward / l3_backward on this plan records a pair of
 * HIP events around each stage, on the call's stream. l3_timing_read waits
 * for those events and returns, per stage, the summed milliseconds and the
 * number of recorded launches since the last read, then forgets them.
 *   ms, count  host arrays of max_stages entries (either may be NULL)
 *   n_stages   host int; receives the number of stage slots
 * Stage names come from l3_stage_name.
 */
l3_status l3_timing_enable(l3_plan_t plan, int enable);
l3_status l3_timing_read(l3_plan_t plan, double* ms, int64_t* count,
                         int max_stages, int* n_stages);
const char* l3_stage_name(int stage);

#ifdef __cplusplus
}
#endif
#endif /* L3_H */
