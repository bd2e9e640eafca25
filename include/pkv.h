/*
 * pkv.h -- C ABI of the MI355X paged-KV attention library (libpkv.so).
 *
 * What the library computes (the FlashInfer pages are the source):
 *   - batched attention over a paged KV cache: the cache lives in fixed-size
 *     pages that need not be contiguous, and a page table lists each
 *     request's pages (article "FlashInfer", section "Block-sparse cache
 *     representation"; docs index "KV-Cache Layout in FlashInfer" >
 *     "Page Table Layout", "Layout: NHD/HND");
 *   - decode (one query token per request) and causal prefill / append (many
 *     query tokens per request appended after a cached prefix), exact
 *     softmax attention with a running maximum (article "FlashInfer",
 *     sections "Correctness and numerical behavior" and "Extreme-negative-logit
 *     correction"; docs index "flashinfer.decode", "flashinfer.prefill");
 *   - every output row comes with its log-sum-exp, forming an attention
 *     state; states of disjoint KV parts merge into the state of their union
 *     (article "FlashInfer", section "Attention states"; docs index
 *     "flashinfer.cascade" > "Merge Attention States", "Cascade Attention");
 *   - a host-side plan that inspects lengths and splits the KV into work
 *     chunks, and a run that reuses the plan with stable workspace buffers
 *     (article "FlashInfer", section "Plan and run").
 *
 * Conventions used by every entry point:
 *   - Device pointers come from the caller (e.g. torch allocations); the
 *     library never allocates or frees memory and keeps no pointer past the
 *     call, except the workspace pointers a plan records (see pkv_plan_info).
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream). Run
 *     and merge calls are asynchronous on that stream and do no host sync.
 *   - Run, merge, single-decode (given its workspace) and append calls
 *     launch a fixed sequence of kernels with no allocation, no memset and
 *     no host synchronisation, so they may be captured into a HIP graph on
 *     the stream and replayed: a replay reads whatever the captured buffers
 *     hold at that time (the plan's workspaces must stay as they were). The
 *     *_timed variants are excluded (their events belong to the caller).
 *   - Layouts are row-major and contiguous unless strides are given:
 *       q, o     : decode [batch, num_qo_heads, head_dim],
 *                  prefill [total_qo_tokens, num_qo_heads, head_dim];
 *       lse      : float32, natural log, [rows, num_qo_heads];
 *       KV pages : element (page, slot, kv_head, d) at
 *                  base + page*page_stride + slot*token_stride + kv_head*head_stride + d,
 *                  so both page layouts of the docs index ("Layout: NHD/HND") are
 *                  described by strides: NHD token_stride = Hkv*head_dim,
 *                  head_stride = head_dim; HND token_stride = head_dim,
 *                  head_stride = page_size*head_dim.
 *   - Page tables are int32: kv_indptr[batch+1] (monotone), kv_indices[...]
 *     (page ids), last_page_len[batch] (1..page_size for a request with
 *     pages, 0 for a request with none). Request b holds
 *     L_b = (n_b-1)*page_size + last_page_len[b] tokens, token t at page
 *     kv_indices[kv_indptr[b] + t/page_size], slot t%page_size.
 *   - GQA: query head h reads KV head h / G, G = num_qo_heads / num_kv_heads.
 *   - A row that sees no key (empty request, fully masked row) yields O = 0
 *     and LSE = -inf; -inf is never replaced by a finite sentinel.
 *   - sm_scale (the factor on q.k) must be finite and positive.
 *   - Errors: every entry point returns a pkv_status; on failure nothing is
 *     launched and pkv_last_error() returns a thread-local message.
 *
 * Supported today: head_dim 128; fp16 and bf16 storage; fp32 accumulation.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 4

typedef int32_t pkv_status;
enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,         /* malformed argument (pointer, length, table)   */
  PKV_ERR_UNSUPPORTED = 2,         /* well-formed but not implemented (head_dim...)  */
  PKV_ERR_WORKSPACE_TOO_SMALL = 3, /* required sizes are reported in pkv_plan_info   */
  PKV_ERR_PLAN_MISMATCH = 4,       /* plan does not belong to this call's geometry   */
  PKV_ERR_HIP = 5                  /* a HIP runtime call failed                      */
};

typedef int32_t pkv_dtype;
enum { PKV_F16 = 0, PKV_BF16 = 1, PKV_F32 = 2 };

typedef int32_t pkv_kind;
enum {
  PKV_KIND_DECODE = 1,
  PKV_KIND_PREFILL = 2,
  PKV_KIND_CASCADE = 3,
  PKV_KIND_BLOCK_SPARSE = 4,
  PKV_KIND_POD = 5
};

/* A paged K/V cache. k and v are separate device bases with one set of
 * strides (in elements), which also covers an interleaved [pages, 2, P, H, D]
 * pool. head_dim elements of one (page, slot, head) are contiguous. All
 * strides must be multiples of 8 elements and k, v 16-byte aligned;
 * token_stride is below 2^26 and page_stride below 2^30 elements (the kernels
 * form a page's byte offset in 32 bits and multiply it by the page id in 64).
 * Otherwise the run calls return PKV_ERR_INVALID_ARG. */
typedef struct pkv_paged_kv {
  const void* k;
  const void* v;
  int64_t page_stride;
  int64_t token_stride;
  int64_t head_stride;
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  pkv_dtype dtype; /* PKV_F16 or PKV_BF16 */
} pkv_paged_kv;

/* Attention variants of batch decode and prefill. The FlashInfer article
 * (section "Custom attention templates") lists sliding windows, attention
 * sinks and logit soft caps among the choices a model makes around the
 * query-key product; the pages give no formulas, so these are this library's
 * definitions:
 *   window_left   W >= 0: a query at position p of its request's KV
 *                 (prefill: p = i + L_b - Q_b; decode: p = L_b - 1) sees only
 *                 keys t >= p - W (with the causal mask also t <= p, so at
 *                 most W + 1 keys). -1: no window. Other values are invalid.
 *                 The plan depends on it (items start at the page holding the
 *                 first row's window start); plan and run must agree.
 *   logits_soft_cap  c > 0: every scaled logit x = sm_scale * q.k becomes
 *                 c * tanh(x / c) before the mask and the softmax. 0: off.
 *                 Must be finite and >= 0.
 *   sinks         device float32 [num_qo_heads] (4-byte aligned) or NULL:
 *                 sinks[h] is the logit (natural log, the units of the capped
 *                 scaled logits) of a virtual key with a zero value that joins
 *                 the softmax of every row of query head h, once:
 *                 O = sum_t e^{x_t} v_t / (e^{sinks[h]} + sum_t e^{x_t}) and
 *                 LSE = ln(e^{sinks[h]} + sum_t e^{x_t}). A row that sees no
 *                 key then gets O = 0 and LSE = sinks[h]; -inf is no sink.
 * A NULL pkv_variant* means all three off. */
typedef struct pkv_variant {
  int32_t window_left;
  float logits_soft_cap;
  const float* sinks;
} pkv_variant;

/* Inputs of the work-chunk rule (see pkv_decode_plan). NULL means
 * pkv_default_sched() of the current device. */
typedef struct pkv_sched {
  int32_t num_cus;          /* compute units the work is spread over          */
  int32_t wg_per_cu;        /* work items per CU the chunk size aims for       */
  int32_t min_chunk_tokens; /* no chunk is shorter than this (rounded to pages) */
} pkv_sched;

/* One planned pass (decode, prefill, or one level of a cascade). Offsets are
 * in bytes from the workspace bases recorded in pkv_plan_info.
 * A split group's chunks write partial states into the float workspace: per
 * row, O (f32 [D], already normalised) and the pair (m, l) in the log2 domain
 * (m: the row's reference exponent, a running maximum of sm_scale * log2(e) *
 * q.k; l: the sum of 2^(x_t - m) over the chunk's keys), so that a merge can
 * weight chunk k by l_k * 2^(m_k - M) with an exact exponent difference; the
 * chunk's natural-log LSE is (m + log2 l) * ln 2. */
typedef struct pkv_plan_part {
  int32_t num_items;        /* work items = workgroups launched              */
  int32_t num_groups;       /* (request, tile, kv head) merge groups          */
  int32_t chunk_pages;      /* chunk size c of the rule, in pages             */
  int32_t rows_per_tile;    /* query rows per item (G for decode, 128 prefill) */
  int32_t num_slots;        /* partial states written by the groups' chunks   */
  int32_t causal;
  int32_t window_left;      /* the sliding window the plan was made for (-1: none) */
  int32_t reserved;
  int64_t items_off;        /* int ws: int32 [num_items][8]                   */
  int64_t groups_off;       /* int ws: int32 [num_groups][8]                  */
  int64_t kv_len_off;       /* int ws: int32 [batch] KV length per request    */
  int64_t part_o_off;       /* float ws: f32 [num_slots][rows_per_tile][D]    */
  int64_t part_ml_off;      /* float ws: f32 [num_slots][rows_per_tile][2] (m, l) */
} pkv_plan_part;

/* A plan: a plain struct the caller owns (copyable, no pointers to free).
 * Valid for any run with the same lengths, heads, page size and dtype, as
 * long as the recorded workspaces stay allocated at the same addresses. */
typedef struct pkv_plan_info {
  uint32_t magic;
  int32_t abi_version;
  pkv_kind kind;
  pkv_dtype dtype;
  int32_t batch;
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t total_qo;          /* prefill: sum of query lengths; decode: batch */
  pkv_sched sched;
  void* int_ws;              /* device int workspace the plan was copied to  */
  void* float_ws;            /* device float workspace for partial states    */
  int64_t int_ws_required;   /* bytes (also set on WORKSPACE_TOO_SMALL)      */
  int64_t float_ws_required; /* bytes (also set on WORKSPACE_TOO_SMALL)      */
  int64_t order_off;         /* POD: int ws offset of the launch order (int32)   */
  int32_t num_blocks;        /* POD: workgroups of the mixed launch              */
  int32_t batch2;            /* POD: decode requests (batch = prefill requests)  */
  pkv_plan_part part[2];     /* part[0]: the pass; cascade: [0] prefix, [1] suffix;
                                POD: [0] prefill, [1] decode */
} pkv_plan_info;

/* Thread-local message of the last failure on this thread ("" if none). */
const char* pkv_last_error(void);

/* PKV_ABI_VERSION of the loaded library. */
int32_t pkv_abi_version(void);

/* sizeof(pkv_plan_info) as compiled into the library (lets a foreign-function
 * binding check its mirror of the struct). */
size_t pkv_plan_info_size(void);

/* Fill *out with defaults for `device`: num_cus = the device's CU count,
 * wg_per_cu = 4, min_chunk_tokens = 128 (below that a chunk's fixed cost
 * outweighs the parallelism it adds). Needs a GPU. */
pkv_status pkv_default_sched(int32_t device, pkv_sched* out);

/* Defaults tuned to one kernel: as pkv_default_sched, but wg_per_cu follows
 * the number of workgroups of that kind's kernel resident on one CU (occ):
 * prefill: occ (one wave of items covers the chip); decode: (5*occ)/2, about
 * two and a half waves of items, so that the longest-first order evens out the
 * last one. A plan given a NULL sched uses this for its own kind (the
 * cascade: decode for level 1, and for level 0 the prefill schedule with
 * wg_per_cu = 1, one item per CU). Needs a GPU. */
pkv_status pkv_default_sched_for(pkv_kind kind, int32_t device, pkv_sched* out);

/* ---------------------------------------------------------------------------
 * Host-only planning (no GPU needed): the work-chunk rule. The FlashInfer
 * article (section "Plan and run") has the plan inspect sequence lengths and
 * cache metadata and pick a schedule that the run then reuses, and notes
 * (section "Purpose and scope") that one fixed schedule spreads uneven
 * requests badly; this rule is this library's schedule.
 *
 * Rule (integer arithmetic, ceil(a/b) rounding up):
 *   rows of request b are GQA-packed (row r = query token r/G, head
 *   g*G + r%G); a tile holds rows_per_tile rows (decode: G; prefill: 128);
 *   a tile's KV extent ends at kv_end = L_b, or with the causal mask
 *   clamp(L_b - Q_b + t_last + 1, 0, L_b) (t_last = query token of its last
 *   row), and starts at kv_lo = 0, or with a sliding window W >= 0
 *   max(0, L_b - Q_b + t_first - W) (t_first = query token of its first row);
 *   p_lo = floor(kv_lo / P), pages(tile) = max(0, ceil(kv_end / P) - p_lo);
 *   work = Hkv * sum pages(tile); target = num_cus * wg_per_cu;
 *   c = max(max(1, ceil(min_chunk_tokens / P)), ceil(work / target));
 *   each (b, tile, g) group splits into max(1, ceil(pages / c)) chunks, chunk
 *   j covering pages [p_lo + j*c, p_lo + min((j+1)*c, pages)) and tokens
 *   [min((p_lo + j*c)*P, kv_end), min((p_lo + (j+1)*c)*P, kv_end)); split
 *   groups get consecutive partial slots in (b, tile, g) order; items run
 *   longest first (descending token count, ties by ascending b, tile, g, j).
 * Outputs: items_out[num_items][8] = {b, g, tile, page_begin, page_end,
 *   kv_begin, kv_end, slot (-1 = writes the final output)};
 *   groups_out[num_groups][8] = {b, tile, g, slot_begin, num_chunks,
 *   base_slot_begin, base_num_chunks, base_row} (the last three are 0 except
 *   in a cascade's suffix part, see pkv_cascade_plan);
 *   counts_out[4] = {num_items, num_groups, chunk_pages, num_slots}.
 * qo_indptr_h may be NULL for decode (kind PKV_KIND_DECODE, one query token
 * per request). window_left as in pkv_variant (-1: none). Returns
 * WORKSPACE_TOO_SMALL (counts still filled) when items_cap / groups_cap are
 * too small.
 * ------------------------------------------------------------------------- */
pkv_status pkv_plan_host(pkv_kind kind, const int32_t* qo_indptr_h, const int32_t* kv_indptr_h,
                         const int32_t* last_page_len_h, int32_t batch, int32_t num_qo_heads,
                         int32_t num_kv_heads, int32_t page_size, int32_t causal,
                         int32_t window_left, const pkv_sched* sched, int32_t* items_out,
                         int32_t items_cap,
                         int32_t* groups_out, int32_t groups_cap, int32_t* counts_out);

/* Workspace sizes (bytes) that suffice for every plan of `kind` with at most
 * `max_items` work items: the stable workspace buffers that the FlashInfer
 * article (section "Plan and run") has a plan fill and every run reuse.
 * Bounds for every plan of `kind` with at most
 * `max_items` work items (for the cascade and the mixed batch: both parts
 * together), whatever the lengths, so a caller can allocate once before
 * planning (graph capture, serving loops). `batch`: requests (decode,
 * prefill), query blocks (block-sparse), suffix requests (cascade), prefill
 * plus decode requests (mixed batch). Sizes follow the plan calls' own
 * layout with max_items items, merge groups and partial-state slots (a plan
 * never has more groups or slots than items), so they are upper bounds; a
 * plan that splits fewer items needs less float workspace. The exact item
 * count of given lengths is counts_out[0] of pkv_plan_host. No GPU call.
 * Errors: INVALID_ARG (NULL outputs, negative sizes, heads not a multiple,
 * unknown kind), UNSUPPORTED (head_dim != 128, G above the kind's limit). */
pkv_status pkv_workspace_size(pkv_kind kind, int32_t batch, int32_t num_qo_heads,
                              int32_t num_kv_heads, int32_t head_dim, int64_t max_items,
                              size_t* int_ws_bytes, size_t* float_ws_bytes,
                              size_t* host_ws_bytes);

/* The plan's work list as the run uses it (the chunk boundaries the FlashInfer
 * article, section "Plan and run", has the plan prepare), for checking and
 * inspection. Copies part `part` (0; or 1, the decode part, for a cascade or
 * mixed-batch plan) of a plan's work list to the caller: items_out[num_items][8] and
 * groups_out[num_groups][8] in the layout of pkv_plan_host (counts in
 * plan->part[part]). Reads the host workspace the plan was made with, which
 * must not have been reused since. No GPU call. Errors: PLAN_MISMATCH (not a
 * plan of this library version), INVALID_ARG (part out of range, NULL
 * buffers where rows exist), WORKSPACE_TOO_SMALL (items_cap / groups_cap
 * below the counts; nothing is written). */
pkv_status pkv_plan_export(const pkv_plan_info* plan, const void* host_ws, int32_t part,
                           int32_t* items_out, int32_t items_cap, int32_t* groups_out,
                           int32_t groups_cap);

/* ---------------------------------------------------------------------------
 * Batch paged decode: one query token per request (docs index
 * "flashinfer.decode" > "Batch Decoding"; the page walk of the FlashInfer
 * article, section "Block-sparse cache representation"; plan and run split as
 * in its section "Plan and run").
 *
 * plan: validates the host page-table copies, applies the rule above, writes
 * the item and group tables into host_ws (pinned memory recommended) and
 * queues one copy of them to int_ws on `stream`, without waiting for it: work
 * queued later on `stream` (the run) sees the tables; work on another stream
 * must be ordered after `stream` first. host_ws must stay allocated and
 * unmodified until that copy has completed. A later plan call (of any kind)
 * given the same host_ws waits for it before writing there, so one staging
 * buffer can serve every plan call; the wait covers only that copy and what
 * was queued on its stream before it. Plan calls that share a host_ws must
 * not run concurrently (from several threads); calls on different host_ws
 * may. The library keeps one HIP event per distinct host_ws it has copied
 * from, for the life of the process. With int_ws / float_ws NULL or too small
 * it returns WORKSPACE_TOO_SMALL, queues nothing and reports the required
 * sizes in *out.
 * run: checks that the plan matches `kv` and launches the decode kernel and,
 * if any group split, the merge kernel (article "FlashInfer", section
 * "Attention states"). Runs of one plan share its workspaces, so they must
 * not overlap: queue them on one stream, or order them. q [batch, Hq, 128],
 * o like q (same dtype as the cache), lse [batch, Hq] float32 or NULL.
 * sm_scale multiplies q.k (usually 1/sqrt(head_dim)).
 * variant (plan: only its window_left is used; run: all of it; NULL = none)
 * selects the attention variants of pkv_variant; the run returns
 * PKV_ERR_PLAN_MISMATCH when its window_left differs from the plan's.
 * Needs 1 <= G <= 16.
 * ------------------------------------------------------------------------- */
pkv_status pkv_decode_plan(const int32_t* kv_indptr_h, const int32_t* last_page_len_h,
                           int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t page_size, pkv_dtype dtype,
                           const pkv_variant* variant, const pkv_sched* sched, void* int_ws,
                           size_t int_ws_bytes, void* float_ws, size_t float_ws_bytes,
                           void* host_ws, size_t host_ws_bytes, void* stream,
                           pkv_plan_info* out);

pkv_status pkv_decode_run(const pkv_plan_info* plan, const void* q, const pkv_paged_kv* kv,
                          const int32_t* kv_indptr_d, const int32_t* kv_indices_d,
                          float sm_scale, const pkv_variant* variant, void* o, float* lse,
                          void* stream);

/* As pkv_decode_run, and times the attention kernel: `attention_start` and
 * `attention_done` (hipEvent_t passed as void*, created by the caller; either
 * may be NULL) ride on the attention kernel's own dispatch (hipExtLaunchKernel),
 * taking its begin and end timestamps, so hipEventElapsedTime between them is
 * that kernel's run time alone (not the queue's dispatch latency, not the
 * merge of split chunks that follows). */
pkv_status pkv_decode_run_timed(const pkv_plan_info* plan, const void* q, const pkv_paged_kv* kv,
                                const int32_t* kv_indptr_d, const int32_t* kv_indices_d,
                                float sm_scale, const pkv_variant* variant, void* o, float* lse,
                                void* stream, void* attention_start, void* attention_done);

/* ---------------------------------------------------------------------------
 * Batch paged prefill / append (docs index "flashinfer.prefill" > "Batch
 * Prefill / Append Attention"; exact attention with the causal mask, article
 * "FlashInfer", sections "Correctness and numerical behavior" and
 * "Extreme-negative-logit correction"): Q_b = qo_indptr[b+1]-qo_indptr[b] query
 * tokens per request, the last Q_b of its L_b keys. causal=1 applies the
 * bottom-right mask: query i sees key t iff t <= i + L_b - Q_b (rows with no
 * visible key give O = 0, LSE = -inf). causal=0 lets every query see all L_b
 * keys. q / o [total_qo, Hq, 128], lse [total_qo, Hq] float32 or NULL.
 * Plan, workspace and variant rules as for decode; the run launches the
 * prefill kernel and, if a group split, a merge kernel for the split groups.
 * Needs G <= 128.
 * ------------------------------------------------------------------------- */
pkv_status pkv_prefill_plan(const int32_t* qo_indptr_h, const int32_t* kv_indptr_h,
                            const int32_t* last_page_len_h, int32_t batch, int32_t num_qo_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                            pkv_dtype dtype, int32_t causal, const pkv_variant* variant,
                            const pkv_sched* sched, void* int_ws, size_t int_ws_bytes,
                            void* float_ws, size_t float_ws_bytes, void* host_ws,
                            size_t host_ws_bytes, void* stream, pkv_plan_info* out);

pkv_status pkv_prefill_run(const pkv_plan_info* plan, const void* q, const pkv_paged_kv* kv,
                           const int32_t* qo_indptr_d, const int32_t* kv_indptr_d,
                           const int32_t* kv_indices_d, float sm_scale,
                           const pkv_variant* variant, void* o, float* lse, void* stream);

/* As pkv_prefill_run, with `attention_start` / `attention_done` on the
 * attention kernel's dispatch (see pkv_decode_run_timed). */
pkv_status pkv_prefill_run_timed(const pkv_plan_info* plan, const void* q, const pkv_paged_kv* kv,
                                 const int32_t* qo_indptr_d, const int32_t* kv_indptr_d,
                                 const int32_t* kv_indices_d, float sm_scale,
                                 const pkv_variant* variant, void* o, float* lse, void* stream,
                                 void* attention_start, void* attention_done);

/* ---------------------------------------------------------------------------
 * Single-request decode over a contiguous NHD cache (the page "FlashInfer: A
 * Kernel Library That Puts Attention, GEMM, and MoE Behind One API", section
 * "Installation Paths", shows single_decode_with_kv_cache as the first call;
 * docs index "flashinfer.decode" > "Single Request Decoding"):
 * k, v [kv_len, Hkv, 128] (token stride Hkv*128), q [Hq, 128] -> o [Hq, 128],
 * lse [Hq] or NULL. The same chunk rule runs on the host with no device
 * tables: chunks are uniform, so items are derived from the workgroup index;
 * a split KV head is merged by a second launch. float_ws holds the partial
 * states: float_ws_required bytes (pass NULL, 0 to query; 0 when nothing
 * splits); calls that share a workspace must not overlap. The contiguous
 * cache is handled as 16-token pages. With kv_len 0, k and v may be NULL
 * (nothing is read) and every row is O = 0, LSE = -inf.
 * ------------------------------------------------------------------------- */
pkv_status pkv_single_decode(const void* q, const void* k, const void* v, int32_t kv_len,
                             int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                             pkv_dtype dtype, float sm_scale, const pkv_sched* sched,
                             void* float_ws, size_t float_ws_bytes, int64_t* float_ws_required,
                             void* o, float* lse, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): as
 * pkv_single_decode, with the partial states in a fixed 32 MiB device array
 * that the library holds on each device it runs on until the process ends,
 * instead of a caller workspace. The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine). Every call on a device shares that
 * device's array: calls that overlap on one device race. The partial states
 * take Hq * 520 B per chunk of the KV; the default sched makes at most about
 * 2048 / Hkv chunks (under 18 MB for G <= 16). A kv_len / sched that needs
 * more than 32 MiB is rejected with PKV_ERR_WORKSPACE_TOO_SMALL. Other errors
 * as pkv_single_decode. */
pkv_status pkv_single_decode_noalloc(const void* q, const void* k, const void* v, int32_t kv_len,
                                     int32_t num_qo_heads, int32_t num_kv_heads,
                                     int32_t head_dim, pkv_dtype dtype, float sm_scale,
                                     const pkv_sched* sched, void* o, float* lse, void* stream);

/* ---------------------------------------------------------------------------
 * Attention-state merges (docs index "Merge Attention States"). For each
 * row: s* = max_k s_k; w_k = exp(s_k - s*); O = sum w_k v_k / sum w_k;
 * LSE = s* + ln(sum w_k); if every s_k is -inf the result is (0, -inf).
 * v_dtype is the dtype of every v array (F16, BF16 or F32); s arrays are
 * float32 natural-log LSEs. Rows are (n, H) pairs of head_dim values.
 * ------------------------------------------------------------------------- */
/* (va, sa) + (vb, sb) -> (vo, so); va, vb, vo [n, H, D]; sa, sb, so [n, H]. */
pkv_status pkv_merge_state(const void* va, const float* sa, const void* vb, const float* sb,
                           void* vo, float* so, int32_t n, int32_t num_heads, int32_t head_dim,
                           pkv_dtype v_dtype, void* stream);

/* (v, s) <- merge((v, s), (v_other, s_other)), in place. */
pkv_status pkv_merge_state_in_place(void* v, float* s, const void* v_other,
                                    const float* s_other, int32_t n, int32_t num_heads,
                                    int32_t head_dim, pkv_dtype v_dtype, void* stream);

/* v [n, K, H, D], s [n, K, H] -> vo [n, H, D], so [n, H]; states merge in
 * ascending k, so results are reproducible bit for bit. */
pkv_status pkv_merge_states(const void* v, const float* s, int32_t n, int32_t num_states,
                            int32_t num_heads, int32_t head_dim, pkv_dtype v_dtype, void* vo,
                            float* so, void* stream);

/* ---------------------------------------------------------------------------
 * Two-level cascade decode (docs index "Cascade Attention",
 * "Multi-level Cascade Inference Data Layout"): `batch` decode requests share
 * one prefix page list (prefix_indices_h/_d, prefix_num_pages pages, the last
 * holding prefix_last_page_len tokens) and each has its own suffix page table.
 * Level 0 computes every request's state over the prefix in one pass that
 * reads the prefix once (all batch*Hq query rows against it, unmasked, the
 * prefix split into chunks) and leaves the chunks' partial states in float_ws;
 * level 1 is a batch decode over the suffixes in which every (request, KV
 * head) group writes partial states, and one merge combines each group's
 * prefix states (base_slot_begin, base_num_chunks, base_row of its group
 * record: the level-0 slots and first row that hold its rows) with its suffix
 * chunks into o [batch, Hq, 128] (cache dtype) and lse [batch, Hq] or NULL.
 * A non-NULL sched applies to both levels; with NULL, level 1 takes the
 * decode default and level 0 the prefill default with wg_per_cu = 1 (see
 * pkv_default_sched_for). Three launches in all. Runs of one plan must not
 * overlap (see pkv_decode_run).
 * ------------------------------------------------------------------------- */
pkv_status pkv_cascade_plan(int32_t prefix_num_pages, int32_t prefix_last_page_len,
                            const int32_t* suffix_indptr_h, const int32_t* suffix_last_page_len_h,
                            int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t page_size, pkv_dtype dtype,
                            const pkv_sched* sched, void* int_ws, size_t int_ws_bytes,
                            void* float_ws, size_t float_ws_bytes, void* host_ws,
                            size_t host_ws_bytes, void* stream, pkv_plan_info* out);

pkv_status pkv_cascade_run(const pkv_plan_info* plan, const void* q, const pkv_paged_kv* kv,
                           const int32_t* prefix_indices_d, const int32_t* suffix_indptr_d,
                           const int32_t* suffix_indices_d, float sm_scale, void* o, float* lse,
                           void* stream);

/* ---------------------------------------------------------------------------
 * Block-sparse attention (docs index "flashinfer.sparse" >
 * "BlockSparseAttentionWrapper"; the block-sparse view of the cache in the
 * FlashInfer article, section "Block-sparse cache representation"). Queries
 * q [num_qo_tokens, Hq, 128] and dense keys / values k, v
 * [num_kv_tokens, Hkv, 128] (contiguous) are cut into blocks of row_block (R)
 * query tokens and col_block (C) key tokens; the mask is a BSR matrix over
 * those blocks: block row i (query tokens iR .. min(iR+R, N_q)-1) sees the
 * key blocks bsr_indices[bsr_indptr[i] .. bsr_indptr[i+1]-1] (strictly
 * ascending; block j holds keys jC .. min(jC+C, N_kv)-1). Every query token of
 * a block row attends, unmasked, to every key of its listed blocks; a row with
 * no block gets O = 0 and LSE = -inf. The output o [num_qo_tokens, Hq, 128]
 * is in the storage dtype, lse [num_qo_tokens, Hq] float32 natural log (or
 * NULL). The paged layout is the R = 1 case: a block row is a request of R
 * query tokens whose pages are its blocks (page_size C over the dense K/V),
 * so the plan and the kernel are the paged prefill's, unmasked.
 * plan validates on the host: num_block_rows = ceil(N_q / R), the indptr
 * monotone from 0, indices ascending within [0, ceil(N_kv / C)); errors as
 * pkv_prefill_plan, plus PKV_ERR_INVALID_ARG for a bad pattern. The plan keeps
 * the query-block offsets in int_ws. run takes the device copies of the BSR
 * arrays (the same values the plan saw).
 * ------------------------------------------------------------------------- */
pkv_status pkv_block_sparse_plan(const int32_t* bsr_indptr_h, const int32_t* bsr_indices_h,
                                 int32_t num_block_rows, int32_t num_qo_tokens,
                                 int32_t num_kv_tokens, int32_t row_block, int32_t col_block,
                                 int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                                 pkv_dtype dtype, const pkv_sched* sched, void* int_ws,
                                 size_t int_ws_bytes, void* float_ws, size_t float_ws_bytes,
                                 void* host_ws, size_t host_ws_bytes, void* stream,
                                 pkv_plan_info* out);

pkv_status pkv_block_sparse_run(const pkv_plan_info* plan, const void* q, const void* k,
                                const void* v, const int32_t* bsr_indptr_d,
                                const int32_t* bsr_indices_d, float sm_scale, void* o, float* lse,
                                void* stream);

/* ---------------------------------------------------------------------------
 * Mixed prefill + decode batch in one launch (POD attention: named in the
 * page "FlashInfer: A Kernel Library That Puts Attention, GEMM, and MoE Behind
 * One API", section "The Feature List: What Is Actually Covered", as the
 * kernel that fuses prefill and decode for mixed batching; docs index
 * "flashinfer.pod" > "PODWithPagedKVCacheWrapper").
 *
 * The results are exactly those of pkv_prefill_run over the prefill requests
 * (causal as given) and pkv_decode_run over the decode requests; both read the
 * same page pools `kv` through their own page tables. plan builds the two
 * parts with the work-chunk rule (part[0] prefill, part[1] decode; sched as in
 * the single-kind plans, each part resolving a NULL sched for its own kind)
 * and an interleaved launch order of their items: an item costs its KV token
 * count + 1, and the next workgroup takes an item from the part whose emitted
 * share of its own total cost is smaller (prefill on ties), so every stretch
 * of the grid mixes MFMA-bound prefill items with HBM-bound decode items. run
 * launches one kernel for all items, then the merges of each part's split
 * groups. Either part may be empty (batch_p = 0 or batch_d = 0).
 * Outputs: o_p [total_qo, Hq, 128] and o_d [batch_d, Hq, 128] in the cache
 * dtype, lse_p / lse_d float32 or NULL. Needs G <= 16. Errors as
 * pkv_prefill_plan / pkv_decode_plan. On WORKSPACE_TOO_SMALL, a host_ws of at
 * least int_ws_required bytes still receives the plan's integer tables (also
 * true of the other plan calls).
 * ------------------------------------------------------------------------- */
pkv_status pkv_pod_plan(const int32_t* qo_indptr_h, const int32_t* kv_indptr_p_h,
                        const int32_t* last_page_len_p_h, int32_t batch_p, int32_t causal,
                        const int32_t* kv_indptr_d_h, const int32_t* last_page_len_d_h,
                        int32_t batch_d, int32_t num_qo_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t page_size, pkv_dtype dtype,
                        const pkv_sched* sched, void* int_ws, size_t int_ws_bytes,
                        void* float_ws, size_t float_ws_bytes, void* host_ws,
                        size_t host_ws_bytes, void* stream, pkv_plan_info* out);

pkv_status pkv_pod_run(const pkv_plan_info* plan, const pkv_paged_kv* kv, const void* q_p,
                       const int32_t* qo_indptr_d, const int32_t* kv_indptr_p_d,
                       const int32_t* kv_indices_p_d, void* o_p, float* lse_p, const void* q_d,
                       const int32_t* kv_indptr_d_d, const int32_t* kv_indices_d_d, void* o_d,
                       float* lse_d, float sm_scale, void* stream);

/* As pkv_pod_run, with `attention_start` / `attention_done` on the mixed
 * kernel's dispatch (the merges are not included; see pkv_decode_run_timed). */
pkv_status pkv_pod_run_timed(const pkv_plan_info* plan, const pkv_paged_kv* kv, const void* q_p,
                             const int32_t* qo_indptr_d, const int32_t* kv_indptr_p_d,
                             const int32_t* kv_indices_p_d, void* o_p, float* lse_p,
                             const void* q_d, const int32_t* kv_indptr_d_d,
                             const int32_t* kv_indices_d_d, void* o_d, float* lse_d,
                             float sm_scale, void* stream, void* attention_start,
                             void* attention_done);

/* ---------------------------------------------------------------------------
 * Appending new K/V rows into a paged cache (docs index "flashinfer.page" >
 * "Append new K/V tensors to Paged KV-Cache"; the page walk is the one of the
 * FlashInfer article, section "Block-sparse cache representation").
 *
 * The page table (kv_indptr, kv_indices, last_page_len, device arrays, int32)
 * already describes the cache *after* the append. Appended row n (n < nnz)
 * names its request b = batch_indices_d[n] and its position t = positions_d[n]
 * within that request; its K row append_k[n] and V row append_v[n] (each
 * [num_kv_heads, 128], contiguous, rows num_kv_heads*128 elements apart) are
 * written to page kv_indices[kv_indptr[b] + t / P], slot t % P, for every KV
 * head, of k_cache and v_cache. Those pools have the NHD layout `layout`
 * describes (its k and v fields are not used). Nothing else is written.
 * A row whose b is outside [0, batch), whose t is outside [0, L_b), or whose
 * page index t / P is not below the request's page count is skipped. Page ids
 * are not range-checked on the device (as for the attention runs).
 * Asynchronous on `stream`; no allocation; element copies are bit-exact.
 * Errors: PKV_ERR_INVALID_ARG for NULL pointers with nnz > 0, nnz or batch
 * < 0, misaligned (16-byte) pointers, bad strides (as pkv_paged_kv);
 * PKV_ERR_UNSUPPORTED for head_dim != 128 or num_kv_heads > 32. */
pkv_status pkv_append_paged_kv(const void* append_k, const void* append_v, int32_t nnz,
                               const int32_t* batch_indices_d, const int32_t* positions_d,
                               void* k_cache, void* v_cache, const pkv_paged_kv* layout,
                               const int32_t* kv_indptr_d, const int32_t* kv_indices_d,
                               const int32_t* last_page_len_d, int32_t batch, void* stream);

/* Host helper for the usual case: request b appends A_b = append_indptr_h[b+1]
 * - append_indptr_h[b] new tokens at the end of its KV (which the page table,
 * after the append, gives as L_b tokens). Fills, for n = append_indptr_h[b] +
 * i, batch_indices_h[n] = b and positions_h[n] = L_b - A_b + i; the output
 * arrays hold append_indptr_h[batch] entries. Host arrays only, no GPU.
 * Errors: PKV_ERR_INVALID_ARG for a page table that pkv_decode_plan would
 * reject, a non-monotone append_indptr_h or append_indptr_h[0] != 0, or
 * A_b > L_b for some b. */
pkv_status pkv_append_positions(const int32_t* append_indptr_h, const int32_t* kv_indptr_h,
                                const int32_t* last_page_len_h, int32_t batch, int32_t page_size,
                                int32_t* batch_indices_h, int32_t* positions_h);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
