/*
 * bsr_attn.h -- C ABI of libbsr_attn: attention over a block-sparse (BSR / paged)
 * KV cache on an AMD Instinct MI355X (gfx950).
 *
 * The interface follows the plan/run ("inspector-executor") split of FlashInfer as
 * the pages describe it: a host-side plan is built once per generation step from the
 * sequence-length information and reused by every layer, and the run calls execute
 * on the GPU from a caller-owned workspace.
 *   - "FlashInfer: A Customizable Attention Engine for LLM Serving", §6 and §8
 *     (plan(indptr, indices, last_page_length, heads, head_dim, page_size) then
 *     run(q, paged_kv_cache) per layer; caller-owned workspace; "NHD" layout).
 *   - "FlashInfer 原理", §⑨-⑩ (plan on the CPU, async copy into the workspace,
 *     persistent kernels follow the plan; plan reused by all layers).
 *   - "FlashInfer: Engineering a Customizable, Block-Sparse Attention Engine for LLM
 *     Inference Serving", §VIII.4-VIII.6 (work queue per CTA plus the partial ->
 *     final reduction map, written to fixed workspace offsets).
 *
 * Conventions shared by every call
 *   - All integer index arrays are int32.  "host" pointers are ordinary CPU memory,
 *     "device" pointers are HIP device memory on the current device.
 *   - Streams are passed as `void*` holding a hipStream_t (NULL = the null stream).
 *     Every GPU call is stream-ordered and never synchronises the host.
 *   - Return value: BSR_OK (0) or a negative bsr_status.  On error nothing was
 *     launched and a message is available from bsr_last_error() (thread-local).
 *     No call aborts or throws across the ABI.  A device fault inside a launched
 *     kernel surfaces at the caller's next synchronisation, as for any HIP kernel.
 *   - The library never allocates device memory: Q, K, V, O, LSE and the workspace
 *     belong to the caller.  It owns only the opaque plan and its pinned staging.
 */
#ifndef BSR_ATTN_H
#define BSR_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bsr_status {
  BSR_OK = 0,
  BSR_INVALID_ARG = -1, /* malformed arrays, null pointers, bad sizes */
  BSR_UNSUPPORTED = -2, /* head_dim / dtype / group size not compiled in */
  BSR_CAPACITY = -3,    /* workspace smaller than the plan needs */
  BSR_HIP_ERROR = -4    /* a HIP runtime call or launch failed */
} bsr_status;

typedef enum bsr_dtype {
  BSR_DTYPE_F32 = 0, /* fp32 storage, fp32 arithmetic */
  BSR_DTYPE_BF16 = 1 /* bf16 storage, bf16 matrix products with fp32 accumulation */
} bsr_dtype;

typedef struct bsr_plan bsr_plan; /* opaque, host-side */

/*
 * Plan description.  BSR view of the KV cache: request i owns the physical pages
 * kv_indices[kv_indptr[i] .. kv_indptr[i+1]) in logical order; its last page holds
 * last_page_len[i] valid tokens, so l_kv(i) = (n_i - 1) * page_size + last_page_len[i]
 * for n_i > 0 pages, 0 otherwise ("FlashInfer 原理" §⑤; "FlashInfer: Making
 * Attention Fit the Serving Workload" §4.1, eq. 7).  Queries are ragged: request i
 * owns query rows qo_indptr[i] .. qo_indptr[i+1]) of Q and O; qo_indptr == NULL means
 * one query per request (decode).
 */
typedef struct bsr_plan_desc {
  int32_t batch;                /* B >= 0 */
  const int32_t* qo_indptr;     /* host int32[B+1] or NULL (decode) */
  const int32_t* kv_indptr;     /* host int32[B+1], kv_indptr[0] = 0, non-decreasing */
  const int32_t* kv_indices;    /* host int32[kv_indptr[B]], each in [0, num_pages); or NULL
                                   for a contiguous cache: request i's pages are kv_indptr[i]
                                   .. kv_indptr[i+1] - 1 of the pool, in order (the identity
                                   table; kv_indptr[B] <= num_pages).  The plan stores that
                                   table like any other, and the decode kernel computes the
                                   page ids instead of loading them (the affine addressing of
                                   "FlashInfer: Engineering a Customizable, Block-Sparse
                                   Attention Engine for LLM Inference Serving" §V.4) */
  const int32_t* last_page_len; /* host int32[B]: in [1, page_size] if n_i > 0, else 0 */
  int32_t num_pages;            /* pool size, for validation of kv_indices */
  int32_t num_qo_heads;         /* H_qo, a multiple of H_kv */
  int32_t num_kv_heads;         /* H_kv >= 1 */
  int32_t head_dim;             /* d */
  int32_t page_size;            /* P >= 1 (tokens per page; 1 = vector sparse);
                                   P * num_kv_heads * head_dim < 2^31 */
  int32_t causal;               /* 1: key k visible to query q iff k <= q + l_kv - l_qo */
  int32_t num_workers;          /* C: persistent workers; 0 => default for 256 CUs */
  int32_t tile_q;               /* packed query rows per tile; 0 => tile rule */
  int32_t alpha, beta;          /* item cost = alpha * (query positions of its tile) +
                                   beta * chunk_len; both 0 => (2, 1) */
  int32_t window_size;          /* sliding window, in keys: 0 = none (so a zero-filled
                                   description asks for no window); s >= 1 => key k is
                                   visible to query q only if k + l_qo + (s - 1) >= l_kv + q,
                                   i.e. the s keys that end at q's aligned position
                                   ("FlashInfer 原理" §⑧, the mask of the window variant,
                                   whose window_left is s - 1).  Combines with causal, which
                                   supplies the upper bound.  Negative values are
                                   BSR_INVALID_ARG. */
  float logits_soft_cap;        /* 0 = none; c > 0 => every score s = sm_scale * q.k is
                                   replaced by c * tanh(s / c) before masking and softmax
                                   ("FlashInfer: Making Attention Fit the Serving Workload"
                                   §5, eq. 8).  Must be finite. */
} bsr_plan_desc;

/*
 * Build a plan: the load-balanced split-KV partition (longest-processing-time
 * greedy) of "FlashInfer: Engineering a Customizable, Block-Sparse Attention Engine
 * for LLM Inference Serving" §VIII.2 and "FlashInfer: Making Attention Fit the
 * Serving Workload" §6.1-6.2 (eqs. 10-11):
 *   g = H_qo / H_kv; packed query length pq_i = l_qo(i) * g (GQA head fusion, eq. 3);
 *   T_q = tile_q or the smallest of {16, 32, 64, 128} >= ceil(sum pq_i / B);
 *   W = sum_i ceil(pq_i / T_q) * l_kv(i);  chunk limit L = max(1, ceil(W / C));
 *   each query tile's visible KV range is cut into chunks of at most L tokens;
 *   with a sliding window a tile's range starts at the window start of its first query
 *   position, and W is the sum of the tiles' windowed range lengths instead;
 *   chunks are stably sorted by length, descending, and each goes to the worker of
 *   least accumulated cost (ties: lower worker id); an item costs alpha times the query
 *   positions of its tile (1 in decode) plus beta times its chunk length (eq. 11).  A tile with one chunk writes its
 *   final output; chunks of split tiles get partial slots, folded in KV order
 *   (deterministic; no atomics in the arithmetic) by the wave that writes a tile's last
 *   slot on the decode kernel (bf16 or E4M3 KV), otherwise by the merge pass.
 * Copies every host array, so the caller may free them on return.  Pure host code:
 * never touches the GPU.  *out receives the plan (NULL on error).
 */
int bsr_plan_create(const bsr_plan_desc* desc, bsr_plan** out);

/*
 * Composable formats: attention of every query over the union of several BSR views ("levels") of
 * one KV pool, the levels' states combined with the merge operator of eq. 6 ("FlashInfer:
 * Engineering a Customizable, Block-Sparse Attention Engine for LLM Inference Serving" §IV.6 and
 * "FlashInfer 原理" §⑤: a shared prefix stored once as a block row of several queries, B_r > 1,
 * private suffixes as ordinary rows; "FlashInfer: Making Attention Fit the Serving Workload"
 * §7.3, eq. 15).
 *   levels[0 .. n_levels-1]: one description per view, over the same queries and the same pool:
 *     equal num_qo_heads, num_kv_heads, head_dim, page_size, num_pages, logits_soft_cap, alpha,
 *     beta; every level's query count (qo_indptr[B], or B when qo_indptr is NULL) is the same
 *     total_q, and query q of a level is query q of Q/O.  Levels are non-causal (causal = 0,
 *     window_size = 0); tile_q and num_workers of the descriptions are ignored.  The group size
 *     H_qo / H_kv must divide 16.
 *   num_workers: C for the whole plan (0 => default).
 * Every level's block rows are cut into query tiles of 16 packed rows and the tiles of all levels
 * are scheduled together by the partition of bsr_plan_create (W = the levels' summed eq. 10 work,
 * one chunk limit, one sorted list, one heap).  Every chunk writes a partial state; the reduction
 * map holds one entry per query that lists its partial rows in every level (levels in order,
 * chunks in KV order), so one merge pass folds levels and chunks (bsr_plan_view: merge_tiles[k] =
 * query k, merge_row_off = the row of that query inside each slot's tile).  Run with
 * bsr_run_prefill (Q/O [total_q, H_qo, d]): one attention launch over all levels, one merge launch.
 * Errors: BSR_INVALID_ARG for NULL pointers, n_levels outside 1 .. 16, a level that
 * bsr_plan_create rejects (the message names the level) or levels that do not match.
 */
int bsr_plan_create_composable(const bsr_plan_desc* levels, int32_t n_levels, int32_t num_workers, bsr_plan** out);

/* Release a plan.  Waits for an in-flight bsr_plan_upload copy of this plan first. */
void bsr_plan_destroy(bsr_plan* plan);

/*
 * Device workspace bytes the plan needs: plan metadata at fixed offsets plus the
 * partial attention states, fp32 [slots][H_kv][T_q][d] outputs and [slots][H_kv][T_q]
 * log-sum-exps.  The number of slots is below 2*C, so the partial storage obeys the
 * bound of "FlashInfer: Making Attention Fit the Serving Workload" §6.5 (eq. 13).
 */
int bsr_plan_workspace_bytes(const bsr_plan* plan, size_t* bytes);

/*
 * Copy the plan metadata (work queue per worker, partial -> final reduction map, request
 * records and the page list) into fixed offsets of `dev_ws` (device, >=
 * bsr_plan_workspace_bytes) on `stream`, asynchronously, from pinned host staging the
 * plan owns: the CPU plans, the copy goes to a fixed workspace offset, and the GPU runs
 * from there ("FlashInfer: Engineering a Customizable, Block-Sparse Attention Engine for
 * LLM Inference Serving" §VIII.4; "FlashInfer: Making Attention Fit the Serving Workload"
 * §6.3, whose serving-step lifecycle copies metadata into fixed workspace sections and
 * orders that copy before the run).
 *   - Ordering: the copy is ordered only on `stream`.  A run call on another stream must
 *     be ordered after it by the caller (an event or stream wait); the run calls do not
 *     wait for the upload themselves.
 *   - The host staging is filled at the first upload and reused; the plan keeps it until
 *     bsr_plan_destroy, which first waits for the last upload's copy.
 *   - Errors: BSR_INVALID_ARG for a NULL plan or workspace; BSR_CAPACITY if ws_bytes is
 *     below bsr_plan_workspace_bytes (nothing is copied); BSR_HIP_ERROR if the pinned
 *     allocation, the copy or the event record fails.
 *   - The run calls must pass the same workspace pointer (they check it).
 */
int bsr_plan_upload(bsr_plan* plan, void* dev_ws, size_t ws_bytes, void* stream);

/*
 * Read-only host view of a plan, for inspection and parity checks: the two outputs of the
 * scheduler, the work queue of every worker and the partial -> final reduction map
 * ("FlashInfer: Engineering a Customizable, Block-Sparse Attention Engine for LLM
 * Inference Serving" §VIII.5, Figure 6: some final outputs come from one partial, others
 * from several), plus the tiles and items they are built from.  Arrays belong to the plan
 * and live until bsr_plan_destroy; nothing is copied.  window_left is the window of the
 * description as keys left of the diagonal (window_size - 1; -1 = no window).  Errors:
 * BSR_INVALID_ARG for a NULL plan or view.
 *   tiles[num_tiles][5]   = {req, row_start, row_end, vis, n_items}, creation order
 *                           (rows are packed GQA rows of the request; vis = visible
 *                           KV length of the tile)
 *   items[num_items][8]   = {req, tile, row_start, row_end, kv_start, kv_len, worker,
 *                           slot}, creation order (request, tile, kv_start ascending);
 *                           slot = -1 when the item writes the final output
 *   queue_ptr[C+1], queue_items[num_items]: worker w runs items
 *                           queue_items[queue_ptr[w] .. queue_ptr[w+1]) in that order
 *   worker_cost[C]        = accumulated predicted cost of each worker
 *   merge_tiles[num_merge]: tiles written by the merge pass (split or empty), creation
 *                           order; merge_ptr[num_merge+1], merge_slots[]: their slots
 *                           in fold order (ascending kv_start)
 *   tile_lo[num_tiles]    = first visible key of each tile (> 0 only with a window)
 */
typedef struct bsr_plan_view {
  int32_t batch, num_qo_heads, num_kv_heads, head_dim, page_size, causal;
  int32_t group_size, tile_q, num_workers, num_slots;
  int64_t total_work, chunk_limit;
  int32_t num_tiles;
  const int32_t* tiles;
  int32_t num_items;
  const int32_t* items;
  const int32_t* queue_ptr;
  const int32_t* queue_items;
  const int64_t* worker_cost;
  int32_t num_merge;
  const int32_t* merge_tiles;
  const int32_t* merge_ptr;
  const int32_t* merge_slots;
  int32_t window_left;
  float logits_soft_cap;
  const int32_t* tile_lo;
  int64_t custom_mask_bits;  /* sum_i l_qo(i) * l_kv(i): bits of a bsr_run_prefill_masked mask */
  /* composable plans (bsr_plan_create_composable); a single-view plan has num_levels 1 */
  int32_t num_levels;
  const int32_t* level_req_start;  /* [num_levels+1]: first flattened request of each level */
  const int32_t* merge_row_off;    /* per merge slot: partial-row offset (composable plans), else NULL */
} bsr_plan_view;

int bsr_plan_export(const bsr_plan* plan, bsr_plan_view* view);

/*
 * Paged decode: one query per request (plan built with qo_indptr == NULL).
 *   q       device [B, H_qo, d]                     dtype
 *   k_cache device [num_pages, page_size, H_kv, d]  dtype ("NHD", d contiguous)
 *   v_cache device [num_pages, page_size, H_kv, d]  dtype
 *   o       device [B, H_qo, d]                     dtype (bf16 rounded to nearest even)
 *   lse     device [B, H_qo] fp32: natural log of the sum of exp(sm_scale * q.k) over
 *           the request's keys; -inf (with O = 0) for a request without keys.
 * Exact attention, eq. 1 of "FlashInfer: Making Attention Fit the Serving Workload"
 * (§2.1), computed tile by tile with the online-softmax recurrence and split across
 * workers as planned; partial states are combined with the merge of eq. 6.  With bf16 on the
 * decode kernel (head_dim 64 or 128, at most 16 query heads per KV head) this is one launch:
 * the wave that writes the last partial state of a split request folds the request's states
 * in the plan's slot order ("FlashInfer: Engineering a Customizable, Block-Sparse Attention
 * Engine for LLM Inference Serving" §VIII.3, §VIII.6), and a merge launch follows only if a
 * request has no keys (its empty state).  Otherwise (fp32, or the tiled kernel) the attention
 * launch is followed by the merge launch whenever the plan split a request.  The result does
 * not depend on which workgroup ran which work item.  sm_scale must be positive and finite
 * (1/sqrt(d) for the standard operator).  The workspace holds the counters the kernels use to
 * hand out work items and to count arrivals (zero between calls, reset by the kernels), so run
 * calls on one workspace must not overlap; calls on different workspaces may.
 */
int bsr_run_decode(const bsr_plan* plan, const void* ws, const void* q, const void* k_cache,
                   const void* v_cache, void* o, float* lse, int32_t dtype, float sm_scale,
                   void* stream);

/*
 * bsr_run_decode without a caller workspace, for callers that cannot allocate device memory
 * (code under graph capture, serving loops, harnesses that forbid allocation).  The workspace is
 * a static device array of the library, at most 32 MiB (plans needing more return BSR_CAPACITY
 * before touching the GPU), which every GPU the library runs on holds until the process ends.
 * Each call copies the plan's metadata into that array on `stream` (from the plan's pinned
 * staging once bsr_plan_upload has created it, else from ordinary host memory, which the HIP
 * runtime copies before returning), then runs the same kernels as bsr_run_decode; the results
 * are identical.  Arguments, layouts and errors are those of bsr_run_decode; the call allocates
 * nothing.  All calls on one GPU share the array and it keeps the last call's contents: calls
 * that overlap on one GPU (other streams, other threads, other plans) race, so order them.
 * Nothing in the array needs clearing between calls.
 */
int bsr_run_decode_scratch(const bsr_plan* plan, const void* q, const void* k_cache, const void* v_cache,
                           void* o, float* lse, int32_t dtype, float sm_scale, void* stream);

/*
 * Paged decode over an E4M3 KV cache: as bsr_run_decode with bf16 Q and O, but k_cache and
 * v_cache hold one byte per element in the OCP 8-bit float "E4M3FN" encoding (sign, 4
 * exponent bits with bias 7, 3 mantissa bits; S.1111.111 is NaN; largest finite 448) and
 * every stored value stands for value * k_scale (K) or value * v_scale (V), one scale per
 * tensor.  Layout [num_pages, page_size, H_kv, d] bytes, "NHD".  Decode with an e4m3 KV
 * cache is the configuration of the vLLM integration in "FlashInfer: Making Attention Fit
 * the Serving Workload" (Appendix G.4, Table 8); the pages leave the encoding and scaling
 * open, and this is the OCP format with per-tensor scales.  k_scale and v_scale must be
 * positive and finite.  Supported where the bf16 decode kernel is (head_dim 64 or 128, at
 * most 16 query heads per KV head), else BSR_UNSUPPORTED.  Reads half the KV bytes of bf16.
 * As with bsr_run_decode, split requests are folded inside the attention kernel, so the call
 * is one launch unless a request has no keys.
 */
int bsr_run_decode_e4m3(const bsr_plan* plan, const void* ws, const void* q, const void* k_cache,
                        const void* v_cache, void* o, float* lse, float sm_scale, float k_scale,
                        float v_scale, void* stream);

/*
 * Ragged (optionally causal) prefill.  Same arguments as bsr_run_decode but Q and O
 * are [qo_indptr[B], H_qo, d] (packed, no padding) and the causal flag comes from the
 * plan.  A non-causal plan whose "requests" are groups of queries sharing pages is
 * the shared-prefix level of the composable format.
 */
int bsr_run_prefill(const bsr_plan* plan, const void* ws, const void* q, const void* k_cache,
                    const void* v_cache, void* o, float* lse, int32_t dtype, float sm_scale,
                    void* stream);

/*
 * bsr_run_prefill with a custom mask (any plan, decode or prefill): the LogitsMask variant of
 * "FlashInfer: Engineering a Customizable, Block-Sparse Attention Engine for LLM Inference
 * Serving" §VII (tree attention and importance masks, §III.1), one boolean per (query, key)
 * of each request.  mask: device bytes, the requests' [l_qo, l_kv] boolean matrices in
 * request order, each row-major, packed 8 per byte with bit b of the whole string at bit
 * b mod 8 of byte b / 8 (the pages fix no storage format); request i starts at bit
 * sum_{r<i} l_qo(r) l_kv(r), and the buffer holds at least ceil(custom_mask_bits / 8) bytes
 * (bsr_plan_view).  A key takes part only if its bit is set and the plan's causal and
 * window predicates allow it; a query row left with no key is the empty state (O = 0,
 * LSE = -inf).  The plan's work partition is unchanged (fully masked chunks are computed
 * and contribute nothing).  bf16 runs use the 4-wave tiled kernel; they are slower than
 * unmasked runs (every block reads its bits).  mask may be NULL only if custom_mask_bits is 0.
 */
int bsr_run_prefill_masked(const bsr_plan* plan, const void* ws, const void* q, const void* k_cache,
                           const void* v_cache, const void* mask, void* o, float* lse, int32_t dtype,
                           float sm_scale, void* stream);

/*
 * (O_a, LSE_a) (+) (O_b, LSE_b) for `rows` x `heads` states of dimension head_dim
 * (eq. 6 and Algorithm 1 of "FlashInfer: Making Attention Fit the Serving Workload",
 * §3.2-3.3).  O: device [rows, heads, head_dim] in dtype; LSE: device fp32
 * [rows, heads], natural log.  A state with LSE = -inf is empty and acts as the
 * identity; two empty states give O = 0, LSE = -inf.  o_out/lse_out may alias o_a/lse_a
 * (in place) or o_b/lse_b.
 */
int bsr_merge_state(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                    void* o_out, float* lse_out, int64_t rows, int32_t heads, int32_t head_dim,
                    int32_t dtype, void* stream);

/*
 * Debug: physical row id (page * page_size + offset, eq. 7) of every logical token of
 * every request, request after request, computed on the GPU by the kernels' own
 * address function.  rows_dev: device int64[sum_i l_kv(i)].
 */
int bsr_debug_gather_rows(const bsr_plan* plan, const void* ws, int64_t* rows_dev, void* stream);

/*
 * Optional per-kernel timing with HIP events recorded on the launch stream around
 * each attention and merge kernel.  bsr_timing_enable(1) starts recording (and clears
 * the totals); bsr_timing_read synchronises on the last recorded event and returns the
 * summed milliseconds and launch counts since enabling.  Off by default.
 */
int bsr_timing_enable(int32_t on);
int bsr_timing_read(double* attn_ms, int64_t* attn_launches, double* merge_ms,
                    int64_t* merge_launches);

/* Workers that keep every workgroup of the kernel resident on `device`
 * (kind 0 = decode, 1 = prefill), for bsr_plan_desc.num_workers. */
int bsr_query_num_workers(int32_t device, int32_t kind, int32_t num_qo_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t* out);

const char* bsr_last_error(void);
const char* bsr_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BSR_ATTN_H */
