/*
 * orca.h - C ABI of liborca.so: one Orca iteration over an arbitrary mixed
 * batch, computed by selective batching, on one MI355X (gfx950).
 *
 * Sources of the operations (page, section):
 *   [houmin]      garden.houmin.site/infra/orca - 3.1.1 iteration-level
 *                 scheduling; 3.1.2 selective batching.
 *   [0h-n0]       0h-n0.github.io Orca digest - "Selective Batching",
 *                 "Scheduler algorithm", "Implementation notes".
 *   [arcsin2]     unpurerationalist.github.io ORCA notes - 3.2, 4.1, 4.2.
 *   [ultralytics] ultralytics.com glossary "Continuous Batching" - limits
 *                 (per-step token cap).
 *
 * Conventions for every entry point
 *   - Sizes are element counts unless a name ends in _bytes.
 *   - "device" pointers are HIP device memory owned by the caller; the
 *     library only borrows them and never frees them.  "host" pointers are
 *     read during the call only.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     GPU entry points only enqueue work on it and never synchronise it;
 *     their results are valid once the stream has reached that point.
 *   - Every argument is validated on the host before anything is enqueued;
 *     a failed check returns ORCA_ERR_INVALID (or ORCA_ERR_UNSUPPORTED for a
 *     shape the kernels do not implement) and has no side effect.
 *     orca_last_error() then describes the failure.
 *   - A HIP runtime failure while enqueuing returns ORCA_ERR_HIP.
 *   - Handles are not thread-safe: one context per stream / thread.
 *
 * Data types.  ORCA_F32: fp32 everywhere.  ORCA_BF16: bf16 storage for
 * weights, activations and the K/V pool; fp32 accumulation in every
 * contraction, fp32 LayerNorm statistics, fp32 softmax, an fp32 residual
 * stream inside the iteration; values are rounded to nearest-even at each
 * bf16 store.
 */
#ifndef ORCA_H
#define ORCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ORCA_OK = 0,
  ORCA_ERR_INVALID = 1,     /* bad argument / descriptor; nothing enqueued */
  ORCA_ERR_NOSPACE = 2,     /* K/V allocator: no contiguous range large enough */
  ORCA_ERR_HIP = 3,         /* the HIP runtime reported an error */
  ORCA_ERR_UNSUPPORTED = 4  /* valid, but a shape the kernels do not cover */
} orca_status;

typedef enum { ORCA_F32 = 0, ORCA_BF16 = 1 } orca_dtype;

/* [houmin] 3.1.2: a request is in the initiation phase while the K/V manager
 * holds no cache for it (all prompt tokens are processed at once), and in
 * the increment phase afterwards (one token per iteration). */
typedef enum { ORCA_INITIATION = 0, ORCA_INCREMENT = 1 } orca_phase;

/* Human-readable name of a status code (static storage). */
const char* orca_status_str(orca_status s);

/* Description of the last failure on the calling thread ("" if none). */
const char* orca_last_error(void);

/* ------------------------------------------------------------------------
 * Attention K/V manager: token-granular allocator over one K/V pool
 * ([0h-n0] implementation notes: the pool is allocated once at start-up
 * because dynamic device malloc/free is too slow; an index table records
 * where each request's entries live; [houmin] 3.1.1: entries are released
 * as soon as a request finishes).  Host memory only; no GPU call.
 * ---------------------------------------------------------------------- */
typedef struct orca_kv orca_kv;

/* New allocator over token slots [0, capacity).  capacity >= 0. */
orca_status orca_kv_create(int64_t capacity, orca_kv** out);
void        orca_kv_destroy(orca_kv* kv);

/* Reserve n_tokens >= 1 contiguous slots at the lowest base that fits
 * (first fit).  *out_base receives the base.  ORCA_ERR_NOSPACE if no free
 * range is large enough (the state is unchanged). */
orca_status orca_kv_alloc(orca_kv* kv, int64_t n_tokens, int64_t* out_base);

/* Release the reservation that starts at `base`; the freed range coalesces
 * with free neighbours.  ORCA_ERR_INVALID if `base` starts no reservation. */
orca_status orca_kv_free(orca_kv* kv, int64_t base);

/* Slots currently reserved, and the capacity. */
int64_t orca_kv_used(const orca_kv* kv);
int64_t orca_kv_capacity(const orca_kv* kv);

/* Length of the reservation starting at `base`, or -1 if there is none. */
int64_t orca_kv_reservation(const orca_kv* kv, int64_t base);

/* ------------------------------------------------------------------------
 * Engine: the model, its K/V pool and one iteration.
 * ---------------------------------------------------------------------- */

/* Decoder shape.  head dim d = hidden / heads.  Supported: hidden % 64 == 0,
 * ffn % 64 == 0; bf16 needs d in {64, 128}; fp32 needs d in {16, 32, 64, 128}. */
typedef struct {
  int32_t layers;
  int32_t hidden;       /* H */
  int32_t heads;
  int32_t ffn;          /* F */
  int32_t dtype;        /* orca_dtype */
  float   ln_eps;       /* LayerNorm epsilon (inside the square root) */
  int64_t kv_capacity;  /* token slots per layer and head in the K/V pool */
} orca_model_desc;

/* One layer's parameters, device pointers of the model dtype.  The block is
 * a pre-LayerNorm decoder layer ([houmin] 3.1.2 lists LayerNorm, the QKV
 * projection, attention, the output projection, GeLU and residual adds):
 *   a  = LN(x; ln1_g, ln1_b)
 *   [q|k|v] = a W_qkv^T + b_qkv      W_qkv [3H][H]: rows 0..H-1 produce Q,
 *                                    H..2H-1 K, 2H..3H-1 V; head h owns
 *                                    columns h*d .. h*d+d-1 of each block
 *   o  = per-request attention of q over the request's own K/V
 *   h1 = x + o W_o^T + b_o           W_o [H][H]
 *   c  = LN(h1; ln2_g, ln2_b)
 *   f  = GeLU_tanh(c W_1^T + b_1)    W_1 [F][H]
 *   y  = h1 + f W_2^T + b_2          W_2 [H][F]
 * Every W is stored row-major [out][in]; vectors are [out]. */
typedef struct {
  const void *ln1_g, *ln1_b, *w_qkv, *b_qkv, *w_o, *b_o;
  const void *ln2_g, *ln2_b, *w_1, *b_1, *w_2, *b_2;
} orca_layer_weights;

/* One request of the batch ([arcsin2] 4.1: the engine receives per request
 * its id, token index and phase).  Host memory.
 *   q_offset, q_len  rows [q_offset, q_offset+q_len) of the flattened
 *                    [sum L, H] input; offsets must be contiguous from 0
 *   kv_len           K/V entries cached before this iteration
 *   phase            ORCA_INITIATION: prompt rows; kv_len == 0 for a whole
 *                    prompt, or the tokens earlier chunks of the same prompt
 *                    cached when a prompt is split over iterations (chunked
 *                    prefill: [ultralytics] limits and combined techniques);
 *                    ORCA_INCREMENT: one new token over its cache
 *                    (kv_len >= 1, q_len == 1)
 *   kv_base          first pool slot of the request's reservation; its
 *                    entry t lives in slot kv_base + t; this iteration
 *                    appends slots kv_base+kv_len .. kv_base+kv_len+q_len-1 */
typedef struct {
  int32_t q_offset;
  int32_t q_len;
  int32_t kv_len;
  int32_t phase;
  int64_t kv_base;
} orca_req_desc;

typedef struct orca_ctx orca_ctx;

/* Create an engine.
 *   desc        model shape (copied)
 *   layers      host array [desc->layers] of device weight pointers (copied;
 *               the weights themselves are borrowed)
 *   kv_pool     device [layers][heads][kv_capacity][2][d] of the model dtype
 *               (borrowed): entry t of head h of a request at layer l has
 *               its key at kv_pool[l][h][kv_base + t][0][0..d-1] and its
 *               value right after it, at [1][0..d-1].  A slot's key and
 *               value rows are adjacent, so the attention over a request's
 *               cache reads one contiguous stream per head, not two
 *   kv          optional (may be NULL) allocator whose capacity equals
 *               desc->kv_capacity; when given, every request's range
 *               kv_base .. kv_base+kv_len+q_len-1 must lie inside one of its
 *               reservations (borrowed; must outlive the context)
 *   max_rows,
 *   max_reqs    largest sum L and request count any iteration will use;
 *               they size the workspace and the pinned metadata buffers
 * Allocates pinned host staging memory (hipHostMalloc); no device memory. */
orca_status orca_create(const orca_model_desc* desc, const orca_layer_weights* layers,
                        void* kv_pool, const orca_kv* kv,
                        int32_t max_rows, int32_t max_reqs, orca_ctx** out);
orca_status orca_destroy(orca_ctx* ctx);

/* Bytes of device workspace an iteration needs (activations, the fp32
 * residual stream, split-attention partials, metadata).  The caller
 * allocates it once; 256-byte alignment is required. */
size_t orca_workspace_bytes(const orca_ctx* ctx);

/* Run one iteration of every layer over the batch ([houmin] 3.1.1: the
 * scheduler invokes the engine for exactly one iteration; 3.1.2: LayerNorm,
 * the four Linear layers, GeLU and residual adds run on the flattened
 * [sum L, H] matrix; attention is split per request and merged back).
 *   reqs, n_reqs  host array of request descriptors (validated, see above)
 *   x             device [sum L][H] model dtype: input rows
 *   y             device [sum L][H] model dtype: output rows of the last
 *                 layer (may not alias x or the workspace)
 *   workspace     device, >= orca_workspace_bytes(ctx) bytes
 * Appends the K/V rows of every request to the pool, at every layer.
 * Metadata goes to the device with one asynchronous copy from a pinned
 * ring of staging buffers; the call does not wait for the GPU except when
 * the ring slot it needs is still being copied from. */
orca_status orca_iteration(orca_ctx* ctx, const orca_req_desc* reqs, int32_t n_reqs,
                           const void* x, void* y, void* workspace, size_t ws_bytes,
                           void* stream);

/* ------------------------------------------------------------------------
 * Measurement: timing events around one step of the layer, in every layer
 * of the iterations that follow.  For throughput accounting of a kernel as
 * it runs inside real iterations (its neighbours, clocks and caches as in
 * production), not needed to run the model.
 * ---------------------------------------------------------------------- */
enum {
  ORCA_STEP_QKV = 0,        /* the QKV Linear with the K/V append */
  ORCA_STEP_ATTENTION = 1,  /* split attention (every request, both phases) */
  ORCA_STEP_OUT_PROJ = 2,   /* output projection + residual (not the LN after it,
                               except fused into a split-K reduce) */
  ORCA_STEP_FFN1 = 3,       /* FFN1 + GeLU */
  ORCA_STEP_FFN2 = 4        /* FFN2 + residual (as ORCA_STEP_OUT_PROJ) */
};

/* Choose the step to time (-1: none).  The first call with a step creates
 * two HIP timing events per layer, owned by the context; every later
 * orca_iteration records them on its stream before and after that step of
 * each layer.  ORCA_ERR_INVALID for an unknown step; ORCA_ERR_HIP if the
 * events cannot be created (timing then stays off). */
orca_status orca_time_step(orca_ctx* ctx, int32_t step);

/* Per-layer milliseconds of the chosen step in the last iteration that ran
 * with it, for layers 0 .. min(n, layers)-1, into host ms[].  Waits for that
 * iteration to finish.  ORCA_ERR_INVALID if no step is chosen or no
 * iteration has run since it was chosen. */
orca_status orca_step_times(orca_ctx* ctx, float* ms, int32_t n);

/* ------------------------------------------------------------------------
 * Single-step entry points: the kernels orca_iteration launches, one step
 * of the layer at a time, with the same launch configuration.  For tests
 * and kernel timing.
 * ---------------------------------------------------------------------- */

/* out[r] = LN(x[r]; gamma, beta) for rows 0..rows-1.  x device fp32
 * [rows][hidden] (the residual stream); gamma, beta device [hidden] and out
 * device [rows][hidden] of `dtype`.  Statistics in fp32, population
 * variance.  ([0h-n0] implementation notes: fused LayerNorm.) */
orca_status orca_op_layernorm(int32_t dtype, const float* x, const void* gamma,
                              const void* beta, void* out, int32_t rows, int32_t hidden,
                              float eps, void* stream);

/* Epilogues of the flattened Linear layers ([houmin] 3.1.2). */
typedef enum {
  ORCA_EPI_BIAS = 0,       /* out[m][n] = acc + bias[n]            (dtype) */
  ORCA_EPI_BIAS_GELU = 1,  /* out[m][n] = GeLU_tanh(acc + bias[n]) (dtype) */
  ORCA_EPI_BIAS_RESID = 2  /* out[m][n] += acc + bias[n]  (out is fp32)    */
} orca_epilogue;

/* acc[m][n] = sum_k a[m][k] * w[n][k] on a device [m][k], w device [n][k],
 * bias device [n] (all `dtype`), then the epilogue.  m >= 0; n % 64 == 0 and
 * k % 64 == 0.  bf16 runs on the MFMA units.
 * workspace: device scratch owned by the caller, may be NULL.  With
 * ws_bytes >= orca_op_linear_workspace_bytes(dtype, m, n, k) > 0 a bf16
 * problem splits K where that pays, writing fp32 partial sums there:
 *   - problems whose output tiles are too few to fill the GPU (chiefly
 *     batches of few rows, made mostly of increment rows: the weights are
 *     streamed once and the arithmetic is light) split every tile;
 *   - large problems whose last round of tiles would leave CUs idle split
 *     only that round's tiles (the rest run unsplit): evenly when the round
 *     is at most half full; fuller, a leading part of each tile's K on one
 *     workgroup and the rest on the CUs the round leaves idle, where the
 *     round shrinks by enough K steps to pay for the partial sums.
 * Otherwise every tile runs over the whole of K and the workspace is not
 * touched.  Every path accumulates in fp32; only the summation order
 * differs.  orca_op_linear_workspace_bytes returns 0 where no split applies
 * (fp32, or tiles that fill whole rounds). */
size_t orca_op_linear_workspace_bytes(int32_t dtype, int32_t m, int32_t n, int32_t k);
/* The kernel form orca_op_linear takes for this problem, without launching
 * anything (host only): the launch planner's choice after the fallbacks,
 * the ORCA_GEMM_VARIANT environment override included.  bf16: 12 and 13 the
 * four-wave 256x256 and 256x192 tiles, 7 the eight-wave 128x128 tile, 6 and
 * 8 the eight-wave 256x256 and 256x192 tiles, 10 split-K (when the call
 * brings orca_op_linear_workspace_bytes of workspace), 0, 3 and 11 pinned
 * forms; -1 for fp32 (the FMA kernel); -2 for shapes orca_op_linear
 * rejects. */
int32_t orca_op_linear_variant(int32_t dtype, int32_t m, int32_t n, int32_t k);
/* The form the prefill (initiation-row) attention of a bf16 model takes for
 * `tiles` 128-query tiles per head over `heads` heads, without launching
 * anything (host only): 64 (64-key steps, two workgroups per CU) or 32
 * (32-key steps, three per CU, taken above two rounds of two-per-CU tiles,
 * heads x tiles > 1024); the ORCA_PF_KEYS environment override (32 or 64)
 * included.  -2 for heads < 1 or tiles < 0.  [houmin] 3.1.2: attention is
 * computed per request; the form only changes how its tiles are scheduled. */
int32_t orca_op_prefill_keys(int32_t heads, int32_t tiles);
/* The workgroup order of the prefill attention launch for a batch of a bf16
 * model with `heads` heads, without launching anything (host only).  The
 * batch's initiation requests (reqs[i].phase == ORCA_INITIATION) each
 * contribute the 128-query tiles of their prompt rows; workgroup j of the
 * launch computes the tile starting at query row q0_out[j] of request
 * req_out[j] (an index into reqs) for head head_out[j].  Up to two rounds of
 * two-per-CU workgroups (tiles x heads <= 1024): the tiles longest-first
 * (by kv_len + last query row), the heads of a tile adjacent.  Beyond that:
 * the tiles of each (request, head) together on one XCD (workgroup j runs
 * on XCD j % 8), so they share its L2.  ORCA_PF_ORDER (0 or 1) pins either.
 * Writes the first min(count, cap) entries (the arrays hold cap entries)
 * and returns count = tiles x heads; -2 for n < 0, heads < 1, cap < 0,
 * a negative q_len or kv_len, or missing arrays.  [houmin] 3.1.2:
 * attention runs per request; the order only decides where and when its
 * tiles run. */
int32_t orca_op_prefill_order(const orca_req_desc* reqs, int32_t n, int32_t heads,
                              int32_t* req_out, int32_t* q0_out, int32_t* head_out, int32_t cap);
orca_status orca_op_linear(int32_t dtype, int32_t epilogue, const void* a, const void* w,
                           const void* bias, void* out, int32_t m, int32_t n, int32_t k,
                           void* workspace, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc): orca_op_linear
 * without the workspace argument.  Its split-K partial sums live in a static
 * device buffer of ORCA_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends (its address is looked up on
 * the first call on each device).  The caller still passes the inputs and
 * the output.  Same kernels, plan and results as orca_op_linear given
 * orca_op_linear_workspace_bytes of workspace.  Calls that overlap on one
 * GPU (two streams or two threads) race on the buffer: serialise them.  No
 * part of the buffer needs to start at zero (a call writes every partial
 * sum it reads), and the last call's contents stay in it.
 * ORCA_ERR_UNSUPPORTED when the few-rows split-K plan of the problem needs
 * more than ORCA_NOALLOC_SCRATCH_BYTES (orca_op_linear_workspace_bytes(dtype,
 * m, n, k) tells in advance); a tiled problem whose split-K tail would need
 * more runs all its tiles over the whole of K instead.  Otherwise as
 * orca_op_linear.  Allocates no memory and calls no allocating routine. */
#define ORCA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
orca_status orca_op_linear_noalloc(int32_t dtype, int32_t epilogue, const void* a, const void* w,
                                   const void* bias, void* out, int32_t m, int32_t n, int32_t k,
                                   void* stream);

/* The fused QKV projection with the K/V manager's append: for every row m,
 * [q|k|v] = a[m] W_qkv^T + b_qkv; q goes to q_out[m][0..H-1]; k and v of
 * head h go to kv_pool_l[h][row_dst[m]][0][..] and kv_pool_l[h][row_dst[m]][1][..].
 * row_dst: device int32 [m], each in [0, kv_capacity).  kv_pool_l points at
 * one layer's pool [heads][kv_capacity][2][d] (the layout of orca_create's
 * kv_pool).  workspace / ws_bytes
 * as for orca_op_linear with n = 3 * hidden, k = hidden.  ([houmin] 3.1.2: the
 * QKV Linear yields 3H columns; the split before attention is index
 * arithmetic; the new K/V of every token is appended to its request.) */
orca_status orca_op_qkv(int32_t dtype, const void* a, const void* w_qkv, const void* b_qkv,
                        void* q_out, void* kv_pool_l, const int32_t* row_dst,
                        int32_t m, int32_t hidden, int32_t heads, int64_t kv_capacity,
                        void* workspace, size_t ws_bytes, void* stream);

/* Split attention of one layer ([houmin] 3.1.2): every request attends
 * separately over its own K/V (initiation: causal over its prompt;
 * increment: one query over kv_len cached entries plus its own new one);
 * outputs land at the request's own rows of o (the merge is index
 * arithmetic).  q, o device [sum L][H] of the context's dtype; the new K/V
 * rows must already be in the pool (orca_op_qkv).  Uses the context's
 * pool at `layer` and its metadata path; workspace as for orca_iteration. */
orca_status orca_op_attention(orca_ctx* ctx, int32_t layer, const orca_req_desc* reqs,
                              int32_t n_reqs, const void* q, void* o, void* workspace,
                              size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Iteration-level scheduler ([houmin] 3.1.1; [0h-n0] scheduler algorithm;
 * [arcsin2] 4.2).  Host only.  Policies: 0 iteration-level, 1 request-level
 * (static) baseline, 2 iteration-level with chunked prefill ([ultralytics]
 * glossary, limits and combined techniques: long prompts are split so
 * prefill does not stall decoding).  Each step:
 *   1. the batch returned by the previous step counts as executed: each
 *      member's kv_len grew by its q_len, and a member whose prompt is then
 *      complete produced one token (a prompt's last chunk yields its first
 *      token);
 *   2. finished (generated == out_len) and cancelled requests leave and
 *      their K/V reservation is released at once (policy 1: a finished
 *      member only when every member of the running batch is through);
 *   3. requests with arrival <= now join the FCFS queue;
 *   4. rows already committed: one per decoding request, then (policy 2)
 *      the next chunk of each prompt still being prefilled, as much as the
 *      token budget leaves, in admission order;
 *   5. FCFS admission while the batch has fewer than max_batch requests:
 *      the head is admitted if its reservation prompt_len + max_tokens fits
 *      the free slot count and a contiguous range exists, and if its prompt
 *      fits the budget left (policy 2: if any budget is left; its first
 *      chunk takes what is left); the first miss ends admission (no
 *      skipping); policy 1 admits only when no batch is running;
 *   6. the batch is emitted: decoding requests (increment, admission
 *      order), continuing prompt chunks, then this step's admissions
 *      (initiation; a chunk after the first has kv_len = prompt tokens
 *      already cached).
 * ---------------------------------------------------------------------- */
typedef struct orca_sched orca_sched;

enum { ORCA_POLICY_ITERATION = 0, ORCA_POLICY_STATIC = 1, ORCA_POLICY_CHUNKED = 2 };

/* kv: the allocator reservations come from (borrowed); its capacity is the
 * scheduler's K/V slot budget. */
orca_status orca_sched_create(orca_kv* kv, int32_t max_batch, int32_t token_budget,
                              int32_t policy, orca_sched** out);
void        orca_sched_destroy(orca_sched* s);

/* Queue a request.  out_len is the output length (the request finishes
 * after producing out_len tokens; the policy never reads it ahead of time).
 * ORCA_ERR_INVALID if the id is taken, a length is < 1, out_len > max_tokens,
 * prompt_len > token_budget (policies 0 and 1) or prompt_len + max_tokens >
 * the K/V capacity. */
orca_status orca_sched_submit(orca_sched* s, int64_t id, double arrival, int32_t prompt_len,
                              int32_t max_tokens, int32_t out_len);

/* One scheduling step at time `now`.  Writes up to `cap` descriptors (host)
 * and their request ids; *n_out = batch size (0: nothing to run now).
 * ORCA_ERR_INVALID if cap < max_batch. */
orca_status orca_sched_step(orca_sched* s, double now, orca_req_desc* out, int64_t* out_ids,
                            int32_t cap, int32_t* n_out);

/* Withdraw a request ([houmin] 3.1.1, scheduling workflow: a cancelled
 * request should leave the batch promptly and free its memory).  A queued
 * request is dropped at once; an admitted one leaves at the next step's
 * eviction (so a batch the engine may still be running is unaffected) and
 * its K/V reservation is released there.  ORCA_ERR_INVALID for an unknown,
 * already released or already cancelled id. */
orca_status orca_sched_cancel(orca_sched* s, int64_t id);

/* 1 when nothing is queued, waiting or running. */
int32_t orca_sched_idle(const orca_sched* s);

/* Earliest arrival not yet queued; ORCA_ERR_INVALID if there is none. */
orca_status orca_sched_next_arrival(const orca_sched* s, double* t);

/* Per-request record: iteration index (0-based, counting non-empty steps)
 * of its initiation, of its last token, and of the step that released it;
 * -1 where not reached.  ORCA_ERR_INVALID for an unknown id. */
orca_status orca_sched_request_info(const orca_sched* s, int64_t id, int64_t* admitted_at,
                                    int64_t* finished_at, int64_t* released_at);

/* Slots reserved by running requests. */
int64_t orca_sched_used(const orca_sched* s);

#ifdef __cplusplus
}
#endif

#endif /* ORCA_H */
