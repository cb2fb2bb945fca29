/*
 * bsk.h -- C ABI of libbsk: batched attention over a paged, block-sparse KV
 * cache for variable-length LLM serving, on AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [FI-paper]   "FLASHINFER: EFFICIENT AND CUSTOMIZABLE ATTENTION ENGINE FOR LLM
 *                INFERENCE SERVING" (blog summary of the FlashInfer paper):
 *                "Research methodology" 1 (block-sparse KV, composable formats),
 *                3 (dynamic load-balanced scheduling: CPU plan, cached on the GPU,
 *                fixed graph-compatible launch); "Results" (fused RoPE kernel,
 *                Streaming-LLM, parallel generation).
 *   [FI-0.6]     "FlashInfer 0.6: JIT compilation, MLA, MoE EP, Blackwell" (wiki):
 *                "Architecture" 1 (block-sparse KV format; page indices prefetched
 *                into on-chip shared memory), "Kernel types" (Decode: query length
 *                1, HBM-bound, GQA; Prefill: compute-bound, chunked prefill; the
 *                Blackwell GQA decode with sliding-window and attention-sink
 *                masking; split-KV).
 *   [FI-PR5329]  "FlashInfer BatchAttention: K/V stride optimisation" (analysis
 *                of PR #5329): "Code analysis" 1 (persistent kernel over two
 *                query-tile classes, 128 and 16 rows, grid from plan_info,
 *                K/V stride comparison, cudaError_t status) and 2 (plan()/run()
 *                with float and int workspace buffers, q, kv cache, out, lse).
 *
 * Conventions
 *   - All memory is owned by the caller.  The library allocates no device
 *     memory and keeps no state except a thread-local error message.
 *   - Device pointers are HIP device addresses; `stream` is a hipStream_t
 *     passed as void* (NULL = the default stream).  Work is enqueued
 *     asynchronously on `stream`; errors found on the host are reported
 *     before anything is enqueued.
 *   - Element strides are in elements (not bytes); the last (head_dim)
 *     dimension of every tensor must be contiguous.
 *   - Every entry point returns a bsk_status; on failure bsk_last_error()
 *     describes it.  No C++ exception crosses this boundary.
 *   - run/merge launches have fixed grids and read all per-step data from
 *     the int workspace, so they can be captured once in a hipGraph and
 *     replayed after each new bsk_plan into the same workspace.
 */
#ifndef BSK_H
#define BSK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t bsk_status;
#define BSK_OK 0
#define BSK_ERR_INVALID_ARG (-1) /* bad argument or inconsistent inputs          */
#define BSK_ERR_UNSUPPORTED (-2) /* valid but not built (head_dim, dtype, ...)    */
#define BSK_ERR_CAPACITY (-3)    /* plan exceeds items/slots/merge capacities     */
#define BSK_ERR_WORKSPACE (-4)   /* a workspace is too small                      */
#define BSK_ERR_HIP (-5)         /* a HIP runtime call failed                     */

#define BSK_DTYPE_F32 0
#define BSK_DTYPE_BF16 1

#define BSK_KV_PAGED 0 /* pools [num_pages, ...], page table per request        */
#define BSK_KV_DENSE 1 /* one contiguous [N, Hk, d] block, token offsets per req */

#define BSK_ROPE_NONE 0
#define BSK_ROPE_STREAMING 1 /* key position = rank in the query's visible set */
#define BSK_ROPE_ABSOLUTE 2  /* key position = token index                     */

/* Device scratch of bsk_run_noalloc, held once per GPU the library runs on. */
#define BSK_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

#define BSK_TILE_DECODE 16       /* query-row tile of bsk_run_decode             */
#define BSK_TILE_PREFILL 128     /* query-row tiles of bsk_run_prefill: 32 rows  */
#define BSK_TILE_PREFILL_256 256 /* per wave, four waves (two workgroups per CU) */
                                 /* or eight (one workgroup per CU)             */

/*
 * Problem description shared by plan, run and merge.  Query rows of a
 * request are its (token i, group member u) pairs flattened as
 * row = i * g + u with g = num_qo_heads / num_kv_heads; q head h*g + u
 * reads kv head h.  The qo_len queries of a request are the last qo_len
 * tokens of its KV sequence (their K/V already appended), so query i sits
 * at position kv_len - qo_len + i, which the causal mask and the sliding
 * window are aligned to.
 */
typedef struct bsk_problem {
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t head_dim;      /* 64 or 128                                          */
  int32_t dtype;         /* q, k, v element type: BSK_DTYPE_F32 or _BF16       */
  int32_t out_dtype;     /* out element type: BSK_DTYPE_F32 or _BF16 (lse f32) */
  int32_t kv_mode;       /* BSK_KV_PAGED or BSK_KV_DENSE                       */
  int32_t page_size;     /* power of two, PAGED only (ignored for DENSE)       */
  int32_t causal;        /* 0/1: key j visible only if j <= query position     */
  int32_t window;        /* > 0: key j visible only if qpos - j < window ...   */
  int32_t sink;          /* ... or j < sink (attention sinks); window <= 0: off */
  int32_t rope_mode;     /* BSK_ROPE_*; rotate-half, q and k both rotated      */
  int32_t fused_merge;   /* 1: run merges split units in-kernel (the chunk that
                            finishes a unit last combines it); 0: run leaves
                            partial states for bsk_merge_states              */
  double rope_theta;     /* RoPE base                                          */
  float sm_scale;        /* logit scale, e.g. 1/sqrt(head_dim)                 */
  /* plan parameters (see bsk_plan) */
  int32_t tile_q;        /* BSK_TILE_DECODE, BSK_TILE_PREFILL or _PREFILL_256  */
  int32_t tile_kv;       /* chunk alignment, multiple of page_size             */
  int32_t num_workers;   /* persistent workgroups = launch grid (> 0)          */
  int32_t split_factor;  /* target chunks per worker (>= 1)                    */
  int32_t min_chunk;     /* lower bound of the chunk length, multiple of tile_kv */
  int32_t max_chunk;     /* upper bound (0: kernel limit), multiple of tile_kv */
  int32_t item_overhead; /* cost added per work item (keys)                    */
  /* capacities (size the workspaces) */
  int32_t max_batch;
  int32_t max_items_per_worker;
  int32_t max_slots;     /* partial-state slots in the float workspace         */
  int32_t max_merge;     /* merge-table entries                                */
  /* K/V stride specialisation ([FI-PR5329]): 0 (default) -- when K and V
     have equal page/head/token strides the bf16 kernels form one address
     per key and reach V through the K-to-V pointer distance; 1 -- always
     use the kernels that address K and V with their own strides */
  int32_t independent_kv_strides;
  /* Two tile classes in one launch ([FI-PR5329, code analysis 1]): 0 (off)
     or BSK_TILE_DECODE with tile_q = BSK_TILE_PREFILL -- requests whose
     qo_len * g rows fit one 16-row tile are planned as decode-class items,
     all others as 128-row items, balanced over the same workers, and
     bsk_run_prefill runs both classes in one persistent launch (bf16,
     paged, no RoPE). */
  int32_t decode_tile_q;
  /* Composable format with a shared prefix ([FI-paper, methodology 1]):
     0 (off) or P > 0 -- every request's KV sequence is a dense prefix of P
     tokens shared by the whole batch (bsk_tensors.prefix_k / prefix_v),
     followed by the request's own paged suffix; kv_len and the page table
     describe the suffix only, the queries are the suffix's last tokens
     (causal within it) and every prefix token is in their past.  The plan
     puts the prefix's 128-row tiles over the batch's query rows and the
     suffixes' decode / 128-row tiles on the same workers, bsk_run_prefill
     runs them in one launch and bsk_merge_states combines each row's prefix
     and suffix partial states.  Needs tile_q 128, decode_tile_q 16, bf16,
     paged suffixes, no window, no RoPE, fused_merge 0. */
  int32_t shared_prefix_len;
} bsk_problem;

/* Filled by bsk_plan; passed unchanged to run/merge. */
typedef struct bsk_plan_info {
  int32_t num_workers;  /* launch grid of bsk_run_*                            */
  int32_t tile_q;
  int32_t batch;
  int32_t num_items;
  int32_t num_slots;
  int32_t num_merge;
  int32_t chunk;        /* chunk length L_c in keys                            */
  int32_t max_kv_len;
  int32_t max_qo_len;
  int32_t max_items_on_worker;
  int64_t total_cost;   /* sum of item costs                                   */
  int64_t max_load;     /* largest per-worker cost                             */
  int64_t used_bytes;   /* bytes of the int workspace written                  */
} bsk_plan_info;

/*
 * Device tensors.  PAGED: k/v are pools addressed as
 *   k[page * k_stride_page + head * k_stride_head + slot * k_stride_tok + c]
 * (e.g. [num_pages, Hk, page_size, d] contiguous: strides Hk*ps*d, ps*d, d);
 * token j of request r lives in page kv_page_indices[kv_indptr[r] + j / page_size],
 * slot j % page_size.  DENSE: token j of request r is
 *   k[(kv_indptr[r] + j) * k_stride_tok + head * k_stride_head + c]
 * (k_stride_page unused).  The same for v with its own strides.
 */
typedef struct bsk_tensors {
  const void* q;          /* [T, Hq, d] in problem.dtype                     */
  int64_t q_stride_tok, q_stride_head;
  const void* k;
  const void* v;
  int64_t k_stride_page, k_stride_head, k_stride_tok;
  int64_t v_stride_page, v_stride_head, v_stride_tok;
  const int32_t* kv_page_indices; /* PAGED only                              */
  void* out;              /* [T, Hq, d] in problem.out_dtype                 */
  int64_t o_stride_tok, o_stride_head;
  float* lse;             /* [T, Hq] natural-log sum-exp of scaled logits    */
  int64_t lse_stride_tok; /* head stride is 1                                */
  const float* rope_cos_sin; /* [rope_n_pos, d/2, 2] (cos, sin), see bsk_rope_table */
  int32_t rope_n_pos;
  int32_t reserved0;
  /* shared dense prefix (problem.shared_prefix_len > 0): token j < P of
     kv head h at prefix_k[j * prefix_k_stride_tok + h * prefix_k_stride_head
     + c], the same for prefix_v with its own strides; NULL otherwise */
  const void* prefix_k;
  const void* prefix_v;
  int64_t prefix_k_stride_tok, prefix_k_stride_head;
  int64_t prefix_v_stride_tok, prefix_v_stride_head;
} bsk_tensors;

/* Human-readable name of a status code (static string). */
const char* bsk_status_string(bsk_status status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* bsk_last_error(void);

/*
 * Persistent-grid size for `problem` on the current device: compute units
 * times the workgroups of the exact kernel variant the problem selects
 * (query-tile class, dtype, head_dim, KV layout, RoPE mode) that fit on one
 * CU at once, at most two for the 16-row decode class (three fit, two were
 * measured faster).  The persistent grid must not exceed what is co-resident (a
 * persistent launch larger than that is what [FI-PR5329, review] reports
 * failing; here it would run a second, unbalanced wave of workers).
 * Only the shape fields of `problem` are read; plan fields may be unset.
 * Needs a GPU.  Errors: INVALID_ARG, UNSUPPORTED, HIP.
 */
bsk_status bsk_device_workers(const bsk_problem* problem, int32_t* num_workers);

/*
 * Workspace sizes for `problem` ([FI-PR5329, code analysis 2]: float and int
 * workspace buffers).  int_ws: plan arrays on the device; host_ws: the same
 * bytes on the host (pinned memory recommended), written by bsk_plan and
 * copied in one transfer; float_ws: max_slots partial states of tile_q rows,
 * each head_dim + 1 floats.  Pure host computation.
 */
bsk_status bsk_workspace_query(const bsk_problem* problem, size_t* int_ws_bytes, size_t* float_ws_bytes,
                               size_t* host_ws_bytes);

/*
 * Build the work plan on the host and upload it ([FI-paper, methodology 3]:
 * runtime lengths -> CPU plan that evenly spreads work over all cores ->
 * cached on the GPU for a fixed launch).  Host inputs:
 *   qo_indptr[batch+1]  query token offsets into q/out/lse,
 *   kv_len[batch]       KV sequence length per request (>= qo_len),
 *   kv_indptr[batch+1]  PAGED: offsets into kv_page_indices;
 *                       DENSE: token offsets into k/v.
 * Each (request, kv head, query tile) is cut into key chunks of L_c =
 * max(min_chunk, roundup(ceil(total_cost * (16 + s) / (16 * num_workers *
 * split_factor)), tile_kv)) keys (s = 1 when tile_q = BSK_TILE_DECODE,
 * else 0; capped by max_chunk) on a grid that starts at the unit's first
 * key rounded down to tile_kv (plus the sink range as its own chunk), and
 * items are assigned longest-first to the least-loaded worker.
 * Multi-chunk units write partial states to float-workspace slots; they
 * are combined in-kernel (problem.fused_merge = 1) or by bsk_merge_states.
 * The exact rules, tie-breaks included, are spelled out at the top of
 * csrc/plan.cpp.
 * host_ws receives the plan; if int_ws_dev is non-NULL its first used_bytes
 * are then copied there on `stream`: by one small kernel that reads host_ws
 * through its device address when host_ws is pinned host memory
 * (hipHostMalloc, torch's pin_memory) and both buffers are 16-byte aligned,
 * else by one hipMemcpyAsync.  host_ws must stay untouched until that copy
 * completes.  int_ws_dev == NULL plans on the host only (no GPU needed).
 * Errors: INVALID_ARG (inconsistent lengths, bad parameters), CAPACITY
 * (more items on a worker, slots or merge entries than allowed),
 * WORKSPACE (buffers too small), HIP.
 */
bsk_status bsk_plan(const bsk_problem* problem, int32_t batch, const int32_t* qo_indptr, const int32_t* kv_len,
                    const int32_t* kv_indptr, void* host_ws, size_t host_ws_bytes, void* int_ws_dev,
                    size_t int_ws_bytes, void* stream, bsk_plan_info* info);

/*
 * The copy half of bsk_plan, for a plan built on the host only (int_ws_dev
 * == NULL there): the first info->used_bytes of host_ws go to int_ws_dev on
 * `stream`, by the same kernel or hipMemcpyAsync as in bsk_plan ([FI-paper,
 * methodology 3]: the CPU plan is copied to the GPU, where a fixed launch
 * reads it).  host_ws must stay untouched until the copy completes, and
 * nothing may read int_ws_dev's previous plan once it is enqueued.
 * host_ws_bytes / int_ws_bytes are the buffers' sizes; used_bytes must fit
 * both.  Errors: INVALID_ARG (null pointers, plan / problem mismatch, a
 * plan size that does not fit), WORKSPACE (int workspace smaller than
 * bsk_workspace_query), HIP.
 */
bsk_status bsk_upload_plan(const bsk_problem* problem, const bsk_plan_info* info, const void* host_ws,
                           size_t host_ws_bytes, void* int_ws_dev, size_t int_ws_bytes, void* stream);

/*
 * Small-tile attention (16 query rows per item): decode ([FI-0.6, kernel
 * types: Decode], query length 1, GQA groups of up to 16 heads) and short
 * multi-token queries.  Persistent kernel: workgroup w runs worker w's items
 * from the int workspace; page ids of an item are staged in LDS; K/V pages
 * are read with coalesced 16-byte loads; logits and P.V use MFMA (bf16) or
 * fp32 MFMA (f32 inputs); online softmax in fp32.  Single-chunk items write
 * out/lse; multi-chunk items write partial (O, LSE) to float_ws, and with
 * problem.fused_merge = 1 the chunk that completes a unit (counted with a
 * device-scope atomic in the int workspace, which the run therefore
 * updates; the counters are back at zero when the run ends) merges it
 * into out/lse.  Concurrent runs must not share one int workspace.
 * RoPE (bf16 only): q and every key are rotated in-kernel from the
 * cos/sin table (K stays unrotated in the cache); STREAMING needs qo_len 1.
 * Errors: INVALID_ARG (plan/tile mismatch, null pointers), UNSUPPORTED
 * (head_dim, dtype, rope with f32), WORKSPACE, HIP (launch failure).
 */
bsk_status bsk_run_decode(const bsk_problem* problem, const bsk_plan_info* info, const bsk_tensors* t,
                          void* int_ws_dev, void* float_ws, size_t float_ws_bytes, void* stream);

/*
 * Large-tile attention (tile_q = 128 or 256 query rows per item): ragged
 * (causal) prefill, including prefill appended after cached KV ([FI-0.6,
 * kernel types: Prefill]) and the dense shared prefix of the composable
 * format ([FI-paper, methodology 1]).  bf16 only; QK^T and PV on bf16 MFMA
 * with fp32 accumulation.  Same output / partial-state contract as
 * bsk_run_decode.  Errors as bsk_run_decode (no RoPE); also INVALID_ARG
 * when a paged page stride exceeds 2^31 - 1 elements.
 */
bsk_status bsk_run_prefill(const bsk_problem* problem, const bsk_plan_info* info, const bsk_tensors* t,
                           void* int_ws_dev, void* float_ws, size_t float_ws_bytes, void* stream);

/*
 * Combine the partial states of every multi-chunk unit of the plan
 * ([FI-0.6, kernel types: split-KV]): per query row,
 * LSE = M + ln sum_c exp(LSE_c - M) with M = max_c LSE_c, and
 * O = sum_c exp(LSE_c - LSE) * O_c, written to t->out / t->lse.  Rows of
 * single-chunk units are left untouched (already written by run).  Needed
 * after a run with problem.fused_merge = 0; after a fused run it recomputes
 * the same values.  float_ws / float_ws_bytes: the workspace the run wrote
 * its partial states to (at least the float size bsk_workspace_query gives
 * for `problem`).  Fixed grid.  Checked on the host before anything is
 * enqueued: the plan must belong to `problem` (same query-tile class and
 * worker count, slots and merge entries within its capacities).
 * Errors: INVALID_ARG (null pointers, plan / problem mismatch, misaligned
 * out), WORKSPACE (float workspace missing or smaller than required), HIP.
 */
bsk_status bsk_merge_states(const bsk_problem* problem, const bsk_plan_info* info, const bsk_tensors* t,
                            const void* int_ws_dev, const void* float_ws, size_t float_ws_bytes, void* stream);

/*
 * bsk_merge_states for one plan's run and bsk_upload_plan for the next plan
 * (built on the host only, for another int workspace) in one launch on
 * `stream`.  [FI-paper, methodology 3] copies the CPU plan to the GPU for a
 * fixed launch; riding that copy on the previous step's merge is this
 * library's addition: with two workspaces in turn, step k's upload then
 * needs no dispatch of its own.  The two parts must touch disjoint memory:
 * the merged plan's first info->used_bytes at int_ws_dev may not overlap
 * the next plan's first next_info->used_bytes at next_int_ws_dev.
 * Arguments problem ..
 * float_ws_bytes are bsk_merge_states', next_problem .. next_int_ws_bytes
 * bsk_upload_plan's, with the same meaning and requirements.  When
 * next_host_ws is not pinned host memory, the merge and a hipMemcpyAsync
 * are enqueued one after the other.  Errors: those of the two calls, and
 * INVALID_ARG when those two plan ranges overlap; every argument is
 * checked before anything is enqueued.
 */
bsk_status bsk_merge_states_upload(const bsk_problem* problem, const bsk_plan_info* info, const bsk_tensors* t,
                                   const void* int_ws_dev, const void* float_ws, size_t float_ws_bytes,
                                   const bsk_problem* next_problem, const bsk_plan_info* next_info,
                                   const void* next_host_ws, size_t next_host_ws_bytes, void* next_int_ws_dev,
                                   size_t next_int_ws_bytes, void* stream);

/*
 * For callers that cannot allocate device memory or hold a float workspace:
 * code under graph capture, tight serving loops, harnesses that forbid
 * allocation.  Runs what bsk_run_decode (problem->tile_q 16) or
 * bsk_run_prefill (128, 256) runs, then, unless problem->fused_merge, what
 * bsk_merge_states runs, with the partial states of split units in a
 * scratch array the library holds in device memory (BSK_NOALLOC_SCRATCH_BYTES
 * per GPU, taken when the library's device code is loaded and kept until the
 * process ends) instead of a caller's float workspace.  Allocates nothing.
 * The scratch layout is fixed per problem shape (slot stride tile_q rows of
 * head_dim + 1 floats), so a captured call stays valid after re-planning.
 * Limit: info->num_slots <= BSK_NOALLOC_SCRATCH_BYTES /
 * (tile_q * (head_dim + 1) * 4), else BSK_ERR_CAPACITY before anything is
 * enqueued.  Every call on one GPU uses the same scratch array, which keeps
 * the last call's partial states (nothing in it needs to start at zero):
 * calls that overlap in time on one GPU (other streams or threads) race, so
 * the caller serialises them.  Outputs, the int workspace contract and the
 * other errors are those of bsk_run_* and bsk_merge_states.
 */
bsk_status bsk_run_noalloc(const bsk_problem* problem, const bsk_plan_info* info, const bsk_tensors* t,
                           void* int_ws_dev, void* stream);

/*
 * Merge two complete states row by row (the composable format's dense
 * prefix state with a sparse suffix state, [FI-paper, methodology 1]):
 * o_a/o_b [rows, head_dim] f32 contiguous, lse_a/lse_b [rows] f32; writes
 * o_out [rows, head_dim] in out_dtype and lse_out [rows].  A row is one
 * (query token, q head) pair: for attention outputs laid out [T, Hq, d]
 * with contiguous heads, rows = T * Hq.  Rows whose two LSEs are both
 * -inf get O = 0, LSE = -inf.  o_out may alias o_a or o_b only when
 * out_dtype is F32.  Errors: INVALID_ARG, HIP.
 */
bsk_status bsk_merge_state_pair(const float* o_a, const float* lse_a, const float* o_b, const float* lse_b,
                                void* o_out, float* lse_out, int32_t rows, int32_t head_dim, int32_t out_dtype,
                                void* stream);

/*
 * Fill the RoPE table used by the fused-RoPE decode ([FI-paper, results:
 * fused RoPE + attention kernel]): table[p][k] = (cos, sin) of
 * p * theta^(-2k/head_dim) for p < n_pos, k < head_dim/2, evaluated in fp64
 * on the device and stored as f32.  table_dev: n_pos * head_dim floats.
 * Errors: INVALID_ARG, HIP.
 */
bsk_status bsk_rope_table(float* table_dev, int32_t n_pos, int32_t head_dim, double theta, void* stream);

/*
 * Append new tokens' K and V to a paged cache, the step before attention
 * in chunked prefill ([FI-0.6, kernel types: Prefill]).  The n_r =
 * append_indptr[r+1] - append_indptr[r] new tokens of request r become the
 * last n_r tokens of its sequence: new token i (rows append_indptr[r] + i
 * of k_new / v_new) is written at logical position kv_len[r] - n_r + i,
 * i.e. page kv_page_indices[kv_page_indptr[r] + pos / page_size], slot
 * pos % page_size ([FI-paper, methodology 1]).  kv_len is the length
 * after the append.
 *   problem: num_kv_heads, head_dim, dtype, page_size (PAGED) are used.
 *   append_indptr [batch+1] (append_indptr[0] = 0, append_indptr[batch] =
 *   n_total), kv_len [batch], kv_page_indptr [batch+1], kv_page_indices:
 *   device int32.
 *   k_new / v_new: device [n_total, num_kv_heads, head_dim] in dtype with
 *   token / head strides new_stride_tok / new_stride_head (elements, the
 *   last dimension contiguous, 16-byte aligned rows).
 *   k_cache / v_cache: the pools, written in place, addressed as in
 *   bsk_tensors with the given page / head / token strides (elements).
 * Tokens whose position falls outside their request's page list (or below
 * 0) are skipped.  The library reads and writes only the named buffers.
 * Errors: INVALID_ARG (null pointers, negative sizes, misaligned
 * pointers or strides, DENSE kv_mode), UNSUPPORTED (head_dim, dtype), HIP.
 */
bsk_status bsk_append_paged_kv(const bsk_problem* problem, int32_t batch, int32_t n_total,
                               const int32_t* append_indptr, const int32_t* kv_len, const int32_t* kv_page_indptr,
                               const int32_t* kv_page_indices, const void* k_new, const void* v_new,
                               int64_t new_stride_tok, int64_t new_stride_head, void* k_cache, void* v_cache,
                               int64_t k_stride_page, int64_t k_stride_head, int64_t k_stride_tok,
                               int64_t v_stride_page, int64_t v_stride_head, int64_t v_stride_tok, void* stream);

/*
 * Unfused RoPE, the reference point of the fused-RoPE decode ([FI-paper,
 * results: fused RoPE + attention kernel]): for every request (one query
 * per request: its last token at kv_len - 1), rotate the keys that query
 * sees -- with problem.window > 0 the window [kv_len - window, kv_len)
 * plus the first problem.sink tokens, else all kv_len keys -- from the
 * paged pool t->k into k_out at the same page slots (same strides as
 * t->k), and rotate the query row (token qo_indptr[r+1] - 1, all q heads)
 * from t->q into q_out.  Positions per problem.rope_mode: STREAMING = rank
 * in the visible set (the query last), ABSOLUTE = token index.  Rotate-half
 * with the table t->rope_cos_sin (bsk_rope_table), fp32 arithmetic, bf16
 * results.  A plain decode (rope_mode NONE, same window/sink) over
 * (q_out, k_out, t->v) then computes the RoPE attention.
 *   qo_indptr [batch+1], kv_len [batch], kv_page_indptr [batch+1]: device
 *   int32; max_kv_len: host bound on kv_len (sizes the grid).
 *   q_out: [tokens, Hq, head_dim] bf16 with strides qo_stride_tok/head.
 * Slots of k_out outside the visible keys are not written.
 * Errors: INVALID_ARG (null pointers, rope_mode NONE, misaligned strides,
 * table shorter than the positions), UNSUPPORTED (dtype not bf16, DENSE,
 * head_dim), HIP.
 */
bsk_status bsk_rope_apply(const bsk_problem* problem, int32_t batch, int32_t max_kv_len, const int32_t* qo_indptr,
                          const int32_t* kv_len, const int32_t* kv_page_indptr, const bsk_tensors* t, void* q_out,
                          int64_t qo_stride_tok, int64_t qo_stride_head, void* k_out, void* stream);

/*
 * Test hook for the block-sparse gather ([FI-0.6, architecture 1]): for
 * every plan item, copy the item's keys [kv_lo, kv_hi) of kv head h,
 * fetched through the same LDS-staged page-id path as the attention
 * kernels, into k_out/v_out (problem.dtype, rows of head_dim) at row
 * offset row_offsets[item_id] (device int64 array indexed by item id).
 * Errors: INVALID_ARG, UNSUPPORTED, HIP.
 */
bsk_status bsk_debug_gather(const bsk_problem* problem, const bsk_plan_info* info, const bsk_tensors* t,
                            const void* int_ws_dev, const int64_t* row_offsets, void* k_out, void* v_out,
                            void* stream);

/*
 * Measurement hook, not part of the method: the device's practical rate for
 * a plain streaming read, the ceiling an HBM-bound kernel such as the decode
 * is compared with.  Reads bytes of src (device memory, 16-byte aligned,
 * bytes a multiple of 16) once, with `grid` workgroups of 256 threads and
 * 16-byte non-temporal loads, and writes one 32-bit word per thread into
 * sink (grid * 256 words, caller-owned): the XOR of the words that thread
 * read, so that the XOR of all of sink equals the XOR of all of src.
 * Errors: INVALID_ARG (null or misaligned pointers, grid outside
 * [1, 2^20], sink too small), HIP.
 */
bsk_status bsk_debug_stream_read(const void* src, size_t bytes, void* sink, size_t sink_bytes, int32_t grid,
                                 void* stream);

/*
 * Measurement hook, not part of the method: the device's practical rate for
 * the paged decode's access pattern.  A page of one kv head's 16 keys is
 * 4 KB of K (or V) at head_dim 128, and a page table scatters pages over the
 * pool, so this reads n_blocks 4 KB blocks of src in the order given by
 * `order` (a device array of n_blocks int32 block indices; an index outside
 * [0, bytes / 4096) is clamped into it), with `grid` workgroups of 256
 * threads, each wave reading whole blocks, two at a time, with 16-byte
 * non-temporal loads.  sink receives one 32-bit word per thread (grid * 256
 * words, caller-owned): the XOR of the words it read, so that for a
 * permutation of all blocks the XOR of all of sink equals that of all of src.
 * src: device memory, 16-byte aligned, bytes a positive multiple of 4096.
 * Errors: INVALID_ARG (null or misaligned pointers, bad sizes, grid outside
 * [1, 2^20], sink too small), HIP.
 */
bsk_status bsk_debug_block_read(const void* src, size_t bytes, const int32_t* order, int32_t n_blocks, void* sink,
                                size_t sink_bytes, int32_t grid, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* BSK_H */
