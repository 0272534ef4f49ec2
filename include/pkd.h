/*
 * pkd.h -- paged GQA decode attention for AMD gfx950 (MI355X), C ABI.
 *
 * The operation: batched decode attention (one query token per request)
 * over a paged KV cache described by a CSR page table, with split-KV load
 * balancing.  It follows the inspector/executor contract of the FlashInfer
 * pages:
 *   - pkd_plan  ("plan"): once per decode step, on the host, from the page
 *     table and head configuration; writes a chunked work schedule into
 *     caller-owned workspaces at fixed addresses (aicassindra "FlashInfer,
 *     in depth", section "Plan and run: the inspector-executor split";
 *     pinghaoyang page, sections on the CUDA-graph conflict and on fixed
 *     pointers);
 *   - pkd_run   ("run"): once per layer, launches the decode kernel and the
 *     merge kernel with fixed grids that read everything else from the
 *     workspace, so a run can be captured in a HIP graph and replayed after
 *     later plans (same sections);
 *   - pkd_merge_state / pkd_merge_states: the exact combine of attention
 *     states (pinghaoyang page, section on why online softmax allows any
 *     split; aicassindra, section "Load balancing with split-KV").
 *
 * Data layouts (all row-major, contiguous):
 *   q         bf16 [batch, num_qo_heads, head_dim]
 *   kv_cache  bf16 [num_pages, 2, page_size, num_kv_heads, head_dim]
 *             (NHD; index 0 of the second axis is K, 1 is V), or the same
 *             shape of FP8 E4M3 codes (one byte each, see pkd_run_scaled)
 *   o         bf16 [batch, num_qo_heads, head_dim]
 *   lse       fp32 [batch, num_qo_heads], natural-log log-sum-exp of the
 *             scaled logits
 *   page table: kv_indptr int32 [batch+1], kv_indices int32 [kv_indptr[batch]],
 *             kv_last_page_len int32 [batch], 1 <= last <= page_size
 *             (aicassindra, section "The block-sparse page table").
 * Query head h attends with KV head h / (num_qo_heads / num_kv_heads).
 *
 * Ownership: the caller owns every buffer (inputs, outputs, the three
 * workspaces).  The library never allocates device memory in pkd_plan,
 * pkd_run or the merge calls.  A workspace must outlive every graph that
 * captured a pkd_run using it.
 *
 * Errors: every call returns a pkd_status; nothing throws across the ABI.
 * pkd_last_error() returns a thread-local message for the last failure.
 *
 * Streams: pkd_stream_t is a hipStream_t (NULL = the null stream).  A plan
 * and the runs that use it must be ordered on the device (same stream, or
 * synchronised by the caller).
 */
#ifndef PKD_H_
#define PKD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkd_handle pkd_handle;
typedef void* pkd_stream_t; /* hipStream_t */

typedef enum pkd_status {
  PKD_OK = 0,
  PKD_ERR_INVALID_ARG = 1,         /* malformed page table or argument */
  PKD_ERR_UNSUPPORTED = 2,         /* head_dim, dtype, layout or page size not built */
  PKD_ERR_DTYPE_MISMATCH = 3,      /* run dtypes differ from the plan's */
  PKD_ERR_WORKSPACE_TOO_SMALL = 4, /* a workspace cannot hold this plan */
  PKD_ERR_STALE_PLAN = 5,          /* run before any plan, or batch differs from the plan */
  PKD_ERR_HIP = 6                  /* a HIP runtime call failed */
} pkd_status;

enum { PKD_DTYPE_BF16 = 1, PKD_DTYPE_FP16 = 2, PKD_DTYPE_FP8_E4M3 = 3 };
enum { PKD_LAYOUT_NHD = 0, PKD_LAYOUT_HND = 1 };

/* Plan kinds (header word PKD_H_KIND). */
enum { PKD_PLAN_DECODE = 0, PKD_PLAN_SHARED = 1 };

/* Device error flags, read with pkd_read_device_error. */
enum { PKD_DEVERR_PAGE_ID = 1 }; /* a kv_indices entry was < 0 or >= num_pages */

/* Scheduling knobs.  A NULL pointer means all defaults. */
typedef struct pkd_plan_opts {
  int32_t fixed_chunk_pages; /* > 0: chunk size in pages (forces splits); 0: derived */
  int32_t min_chunk_tokens;  /* smallest derived chunk, in tokens; <= 0: 128 */
  int32_t alpha;             /* cost = alpha * l_q + beta * chunk_len, l_q = 1; */
  int32_t beta;              /*   alpha < 0 or beta <= 0: 1 */
  int32_t variant;           /* decode kernel for runs of this plan: PKD_VARIANT_* */
  int32_t flags;             /* PKD_PLAN_* flags below (0: none) */
} pkd_plan_opts;

/* Plan flags.  PKD_PLAN_ALL_PARTIALS: every request (every group of a
 * shared-prefix plan) writes its chunks' states as partial states, even a
 * request of one chunk, and the merge list names every request, in request
 * order, so entry r is request row r; pkd_run_composable needs both its
 * plans made this way. */
enum { PKD_PLAN_ALL_PARTIALS = 1 };

/* Decode kernels.  Both compute the same result (to rounding); they differ
 * in where q.k is evaluated. */
enum {
  PKD_VARIANT_AUTO = 0,    /* by measurement: PKD_VARIANT_MFMA_PV for group size 8, pages
                              below 16 tokens or fewer than 768 KV tokens per slot, and for
                              group sizes 3, 5, 6, 7; PKD_VARIANT_MFMA otherwise */
  PKD_VARIANT_DOT2 = 1,    /* q.k with packed bf16 dot products on the vector ALUs (group
                              size 1, 2, 4 or 8) */
  PKD_VARIANT_MFMA = 2,    /* q.k as a 16 x 16 tile on the matrix cores (GQA group as rows),
                              p.v on the vector ALUs (group size 1, 2, 4 or 8) */
  PKD_VARIANT_MFMA_PV = 3  /* both q.k and p.v on the matrix cores (group sizes 1 to 8) */
};

/* ---------------------------------------------------------------------
 * Plan image.  The int workspace (and the output of pkd_plan_host) is an
 * array of int32:
 *   [0, 32)                       device-only words (error flag at 0)
 *   [32, 64)                      header, PKD_H_* below at 32 + index
 *   [off_slots, +S+1)             slot_indptr: items of slot s are
 *                                 items[slot_indptr[s] .. slot_indptr[s+1]);
 *                                 off_slots = 64
 *   [off_first, +8*S)             the first item of each slot again (zeros
 *                                 for a slot without items), so a workgroup
 *                                 can read it without waiting for
 *                                 slot_indptr; off_first = 64 + S + 1
 *                                 rounded up to a multiple of 8
 *   [off_merge, +4*n_split)       off_merge = off_first + 8*S.  Split
 *                                 requests in ascending order: request,
 *                                 first partial id, number of partials, 0
 *   [off_items, +8*I)             off_items = off_merge + 4*n_split rounded
 *                                 up to a multiple of 8.
 *                                 Items, 8 ints each: request, page_begin
 *                                 (index into kv_indices), num_pages,
 *                                 last_len, out (partial id, -1 = write the
 *                                 final output directly), length, id0, id1.
 *                                 id0, id1 are 0 in the image pkd_plan_host
 *                                 returns; in pkd_plan's device copy (items
 *                                 and first-item rows of decode plans) they
 *                                 are the page ids kv_indices[page_begin]
 *                                 and kv_indices[page_begin + 1] (the first
 *                                 twice for a one-page item)
 *   [off_groups, +4*num_groups)   off_groups = off_items + 8*I.
 *                                 Shared-prefix plans only: per group, its
 *                                 first request row, request count, chunk
 *                                 count k and first partial id (-1 when
 *                                 k = 1)
 *   [off_indices, +nnz)           copy of kv_indices taken by pkd_plan
 * In a shared-prefix plan (pkd_plan_shared) the KV rows are groups: an item
 * is one chunk of one group's pages for one row block of its requests
 * (rows_per_block of them) and one KV head, its fields being group,
 * page_begin, num_pages, last_len, out, length, block, head; request r
 * (0-based in the group) of a split group keeps chunk j's state at partial
 * id out + r k, and the merge list has one entry per such request.
 * The float workspace holds the partial states: o_part fp32
 * [n_partials, num_qo_heads, head_dim] followed by lse_part fp32
 * [n_partials, num_qo_heads].
 * ------------------------------------------------------------------- */
enum {
  PKD_H_MAGIC = 0, /* 0x31444B50 */
  PKD_H_VERSION,
  PKD_H_BATCH,
  PKD_H_QO_HEADS,
  PKD_H_KV_HEADS,
  PKD_H_HEAD_DIM,
  PKD_H_PAGE_SIZE,
  PKD_H_SLOTS,
  PKD_H_CHUNK_PAGES,
  PKD_H_ITEMS,
  PKD_H_PARTIALS,
  PKD_H_SPLIT,
  PKD_H_ALPHA,
  PKD_H_BETA,
  PKD_H_NNZ,
  PKD_H_PLAN_ID,
  PKD_H_OFF_SLOTS,
  PKD_H_OFF_ITEMS,
  PKD_H_OFF_MERGE,
  PKD_H_OFF_INDICES,
  PKD_H_TOTAL_TOKENS_LO,
  PKD_H_TOTAL_TOKENS_HI,
  PKD_H_OFF_FIRST,
  PKD_H_KIND,           /* PKD_PLAN_DECODE or PKD_PLAN_SHARED */
  PKD_H_NUM_GROUPS,     /* shared-prefix plans: groups (KV rows) */
  PKD_H_OFF_GROUPS,     /* shared-prefix plans: group table */
  PKD_H_ROWS_PER_BLOCK, /* shared-prefix plans: requests per workgroup (128 / gqa) */
  PKD_H_MIN_CHUNKS,     /* fewest partial states of a merge-list entry (0 if none) */
  PKD_H_MAX_CHUNKS,     /* most partial states of a merge-list entry (0 if none) */
  PKD_H_FLAGS,          /* the plan's PKD_PLAN_* flags */
  PKD_H_COUNT
};
#define PKD_HEADER_BASE 32
#define PKD_PLAN_MAGIC 0x31444B50
#define PKD_PLAN_VERSION 3

/* ------------------------------- handle ------------------------------- */

/* Create a handle bound to HIP device `device`.  `num_slots` is the number
 * of persistent decode workgroups S (the fixed CTA count N_CTA of the
 * pinghaoyang page's chunk bound); 0 picks the compute-unit count times the
 * decode kernel's resident workgroups per unit (one on gfx950), at most 2 per
 * compute unit.  No device memory is allocated. */
int pkd_create(pkd_handle** out, int32_t device, int32_t num_slots);
int pkd_destroy(pkd_handle* h);
int32_t pkd_num_slots(const pkd_handle* h);

/* The decode kernel runs of the handle's current plan launch (PKD_VARIANT_DOT2,
 * _MFMA or _MFMA_PV: PKD_VARIANT_AUTO resolved for the plan's shape); 0
 * before any plan. */
int32_t pkd_planned_variant(const pkd_handle* h);
/* Id of the last successful plan on this handle (0 before any); lets an
 * engine assert that the plan matches its batch (aicassindra, "What to do
 * next", item 3). */
int64_t pkd_plan_id(const pkd_handle* h);
/* The shape the handle's current plan was made for, so a caller can refuse
 * a run whose buffers do not match it before anything is launched (a stale
 * plan ranges from wrong output to out-of-bounds accesses: aicassindra,
 * "Failure modes in production").  Writes 8 ints to shape: requests (rows
 * of q, o and lse), num_qo_heads, num_kv_heads, head_dim, page_size,
 * q_dtype, kv_dtype and the plan kind (PKD_PLAN_*).  PKD_ERR_STALE_PLAN
 * before any plan, PKD_ERR_INVALID_ARG on null pointers. */
int pkd_plan_shape(const pkd_handle* h, int32_t* shape);
const char* pkd_last_error(void);

/* ----------------------------- workspaces ----------------------------- */

/* Bytes each workspace needs for any plan with batch <= max_batch and
 * kv_indptr[batch] <= max_nnz on S = num_slots slots and derived chunk sizes
 * (a plan with fixed_chunk_pages may need more, and is refused with
 * PKD_ERR_WORKSPACE_TOO_SMALL when it does not fit).  Sizing for the worst
 * case is the caller's job (aicassindra, "Failure modes in production",
 * workspace too small).  Returns 0 for invalid arguments. */
size_t pkd_int_workspace_bytes(int32_t max_batch, int32_t max_nnz, int32_t num_slots);
size_t pkd_float_workspace_bytes(int32_t max_batch, int32_t num_slots, int32_t num_qo_heads,
                                 int32_t head_dim);
/* Pinned host staging (allocate with hipHostMalloc or torch pin_memory;
 * pkd_plan rejects memory the device cannot map); it holds two plan images so
 * a new plan never overwrites one whose upload is still in flight. */
size_t pkd_host_workspace_bytes(int32_t max_batch, int32_t num_slots);

/* -------------------------------- plan -------------------------------- */

/* Validate the page table, cut each request's pages into chunks, assign the
 * chunks longest-first to the handle's S slots, and write the schedule
 * (pinghaoyang page, section on splitting long KV then longest-first
 * assignment) into host_workspace; then queue on `stream` one kernel that
 * copies it into int_workspace (reading the pinned host memory directly)
 * together with kv_indices.  kv_indptr and kv_last_page_len are host arrays read during the
 * call; kv_indices is a device array the caller may reuse once `stream` has
 * passed this call.  Built: bf16 q, PKD_LAYOUT_NHD, head_dim 128,
 * num_qo_heads / num_kv_heads from 1 to 8 (PKD_VARIANT_DOT2 and
 * PKD_VARIANT_MFMA: 1, 2, 4 or 8), and either a bf16 cache with
 * page_size in {1, 2, 4, 8, 16, 32, 64} or an FP8 E4M3 cache
 * (kv_dtype PKD_DTYPE_FP8_E4M3, its own matrix-core kernel) with the same
 * page sizes; else PKD_ERR_UNSUPPORTED.  Rejects (PKD_ERR_INVALID_ARG)
 * kv_indptr[0] != 0, a request with no page, last_page_len outside
 * [1, page_size], batch < 1, num_qo_heads not a multiple of num_kv_heads.
 * The workspaces passed here are the ones later runs use. */
int pkd_plan(pkd_handle* h, const int32_t* kv_indptr, const int32_t* kv_indices,
             const int32_t* kv_last_page_len, int32_t batch, int32_t num_qo_heads,
             int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t q_dtype,
             int32_t kv_dtype, int32_t kv_layout, void* int_workspace,
             size_t int_workspace_bytes, void* float_workspace, size_t float_workspace_bytes,
             void* host_workspace, size_t host_workspace_bytes, const pkd_plan_opts* opts,
             pkd_stream_t stream);

/* The same schedule computed on the host only (no HIP call): writes the plan
 * image ints [0, off_indices) described above into `out` (out_bytes long)
 * and stores the number of ints written in *out_ints.  For inspection and
 * tests; kv_indices are not needed. */
int pkd_plan_host(const int32_t* kv_indptr, const int32_t* kv_last_page_len, int32_t batch,
                  int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t page_size, int32_t num_slots, const pkd_plan_opts* opts,
                  int32_t* out, size_t out_bytes, int64_t* out_ints);

/* ------------------------- shared-prefix plans ------------------------- */

/* A shared-prefix (composable) plan: the pinghaoyang page, section
 * "Composable Format：共享前缀与独有后缀分开算", puts a prefix that several
 * requests share in one block row of the KV matrix so that one workgroup
 * reads each prefix page once for all of them (pyshine, "Cascades, Merges,
 * and the Autotuner", describes the same cascade: one pass over the shared
 * prefix serves every request of the group, and each request's suffix
 * state is merged in afterwards).
 *
 * num_groups groups: group g's requests are rows qo_indptr[g] ..
 * qo_indptr[g+1]-1 of q (host int32 [num_groups+1], qo_indptr[0] = 0, every
 * group at least one request) and all attend to group g's pages, given by
 * kv_indptr / kv_indices / kv_last_page_len over groups exactly as for
 * pkd_plan.  Runs of the plan (pkd_run with batch = qo_indptr[num_groups])
 * write, for every request and query head, the attention state over its
 * group's tokens; combine it with the request's own suffix state with
 * pkd_merge_state.
 *
 * Work is cut by the same rule as decode work with the chunk bound counting
 * query tiles (pinghaoyang, section on splitting long KV then longest-first
 * assignment): a row block holds 128 / gqa requests (gqa = num_qo_heads /
 * num_kv_heads), T_eff = sum over groups of row blocks x group tokens,
 * cp = max(ceil(min_chunk_tokens / P), ceil(ceil(T_eff num_kv_heads / S) /
 * P)) pages; an item is one KV head of one (group, row block, chunk) and
 * costs alpha x (requests in its block) + beta x (chunk tokens).  Built for
 * gqa 1, 2, 4, 8 and page_size 16, 32, 64 (else PKD_ERR_UNSUPPORTED), over a
 * bf16 or an FP8 E4M3 cache (runs of an E4M3 plan take per-tensor scales
 * through pkd_run_scaled, as for a decode plan); the variant option is
 * ignored.  Workspaces: size them with pkd_shared_workspace_bytes. */
int pkd_plan_shared(pkd_handle* h, const int32_t* qo_indptr, const int32_t* kv_indptr,
                    const int32_t* kv_indices, const int32_t* kv_last_page_len,
                    int32_t num_groups, int32_t num_qo_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t page_size, int32_t q_dtype, int32_t kv_dtype,
                    int32_t kv_layout, void* int_workspace, size_t int_workspace_bytes,
                    void* float_workspace, size_t float_workspace_bytes, void* host_workspace,
                    size_t host_workspace_bytes, const pkd_plan_opts* opts, pkd_stream_t stream);

/* Workspace sizes for shared-prefix plans of up to max_groups groups over
 * max_batch requests and max_nnz page ids with derived chunks (a forced
 * fixed_chunk_pages may need more; pkd_plan_shared then returns
 * PKD_ERR_WORKSPACE_TOO_SMALL).  Writes the three sizes; returns a status. */
int pkd_shared_workspace_bytes(int32_t max_groups, int32_t max_batch, int32_t max_nnz,
                               int32_t num_slots, int32_t num_qo_heads, int32_t num_kv_heads,
                               int32_t head_dim, size_t* int_bytes, size_t* float_bytes,
                               size_t* host_bytes);

/* The schedule of pkd_plan_shared on the host only, as pkd_plan_host. */
int pkd_plan_shared_host(const int32_t* qo_indptr, const int32_t* kv_indptr,
                         const int32_t* kv_last_page_len, int32_t num_groups,
                         int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t page_size, int32_t num_slots, const pkd_plan_opts* opts,
                         int32_t* out, size_t out_bytes, int64_t* out_ints);

/* ------------------------ plan without workspaces ----------------------- */

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * pkd_plan_static is pkd_plan with its three workspaces replaced by the
 * library's own device array of PKD_STATIC_SCRATCH_BYTES, which every GPU
 * the library runs on holds from the library's load until the process
 * ends: the plan image and the kv_indices snapshot go to its first
 * PKD_STATIC_INT_BYTES, the partial states of split requests to the next
 * PKD_STATIC_FLOAT_BYTES, and the plan image is staged through the last
 * PKD_STATIC_STAGE_BYTES (copied there from the handle's host memory).
 * Nothing is allocated on the device; the handle's host staging (2 x
 * PKD_STATIC_STAGE_BYTES) is allocated on its first static plan and reused.
 * Runs follow with pkd_run / pkd_run_scaled as after pkd_plan, and a run
 * captured in a graph replays correctly after later static plans on the
 * same handle (the regions never move).
 *
 * Limits and sharing: a plan whose image, image plus kv_indices or partial
 * states do not fit their region returns PKD_ERR_WORKSPACE_TOO_SMALL before
 * anything is queued.  The array is shared by every handle and every call
 * on one GPU and keeps the last call's contents, so static plans and their
 * runs on different handles of one GPU must not overlap in time (they would
 * race on the array); a run whose handle's static plan has since been
 * replaced by another handle's returns PKD_ERR_STALE_PLAN (checked on the
 * host at the call, not at graph replay).  A handle's first static plan
 * clears the device error word.  Not under graph capture
 * (PKD_ERR_INVALID_ARG).  Other arguments, errors and ordering rules as
 * pkd_plan; shared-prefix plans need pkd_plan_shared. */
#define PKD_STATIC_INT_BYTES ((size_t)8 << 20)
#define PKD_STATIC_FLOAT_BYTES ((size_t)52 << 20)
#define PKD_STATIC_STAGE_BYTES ((size_t)4 << 20)
#define PKD_STATIC_SCRATCH_BYTES \
  (PKD_STATIC_INT_BYTES + PKD_STATIC_FLOAT_BYTES + PKD_STATIC_STAGE_BYTES)
int pkd_plan_static(pkd_handle* h, const int32_t* kv_indptr, const int32_t* kv_indices,
                    const int32_t* kv_last_page_len, int32_t batch, int32_t num_qo_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t q_dtype,
                    int32_t kv_dtype, int32_t kv_layout, const pkd_plan_opts* opts,
                    pkd_stream_t stream);

/* --------------------------------- run -------------------------------- */

/* Decode attention for the planned batch on one layer's cache: o (and lse
 * when non-NULL) for every request and query head.  Launches exactly two
 * kernels on `stream` with grids fixed by the handle: the decode kernel (S
 * workgroups; the shared-prefix kernel for a plan from pkd_plan_shared) and
 * the merge kernel.  `batch` must equal the planned batch
 * and the dtypes the planned ones (else PKD_ERR_STALE_PLAN /
 * PKD_ERR_DTYPE_MISMATCH).  The buffers must have the planned shape, which
 * this call cannot see through plain pointers and so does not check: q and
 * o [batch, num_qo_heads, head_dim], lse [batch, num_qo_heads] and the
 * cache [num_pages, 2, page_size, num_kv_heads, head_dim] with the plan's
 * num_qo_heads, num_kv_heads, head_dim and page_size (pkd_plan_shape
 * returns them; the Python binding compares every tensor with them and
 * raises before calling here).  Any other shape reads and writes past the
 * buffers.  sm_scale <= 0 means 1/sqrt(head_dim).  A page id
 * outside [0, num_pages) is not read: the kernel uses page 0 instead and
 * raises PKD_DEVERR_PAGE_ID (see pkd_read_device_error). */
int pkd_run(pkd_handle* h, const void* q, int32_t batch, const void* kv_cache,
            int64_t num_pages, int32_t q_dtype, int32_t kv_dtype, void* o, float* lse,
            float sm_scale, pkd_stream_t stream);

/* pkd_run over a cache of FP8 E4M3 codes with one scale per tensor: a K
 * code c stands for e4m3(c) * k_scale and a V code for e4m3(c) * v_scale
 * (OCP E4M3: bias 7, subnormals, no infinities, 0x7F / 0xFF NaN, largest
 * finite 448).  The pinghaoyang page, table of customisable hooks in
 * "可定制注意力模板：把变化留给 JIT" and section "适用边界与工程取舍", treats such a
 * cache as a dequantising key/value transform with a scale contract.  The
 * plan must have been made with kv_dtype PKD_DTYPE_FP8_E4M3.  k_scale and
 * v_scale must be finite and > 0 (else PKD_ERR_INVALID_ARG), and 1 for a
 * bf16 cache.  pkd_run is this call with both scales 1. */
int pkd_run_scaled(pkd_handle* h, const void* q, int32_t batch, const void* kv_cache,
                   int64_t num_pages, int32_t q_dtype, int32_t kv_dtype, void* o, float* lse,
                   float sm_scale, float k_scale, float v_scale, pkd_stream_t stream);

/* The composable format in one call (pinghaoyang page, section "Composable
 * Format：共享前缀与独有后缀分开算": a shared prefix and each request's own
 * suffix are computed apart and their states merged exactly).  `prefix`
 * holds a shared-prefix plan (pkd_plan_shared) over the groups' prefix
 * pages and `suffix` a decode plan (pkd_plan) over each request's own pages,
 * both made with PKD_PLAN_ALL_PARTIALS, for the same `batch` requests, head
 * configuration, page size and dtypes (else PKD_ERR_INVALID_ARG,
 * PKD_ERR_STALE_PLAN or PKD_ERR_DTYPE_MISMATCH, before any launch).  Launches
 * three kernels with fixed grids: the shared-prefix kernel on the prefix
 * plan and the decode kernel on the suffix plan, both writing every chunk's
 * state to their own float workspace, then one merge that combines, for
 * every request and query head, the prefix chunks' states and then the
 * suffix chunks' states into o (bf16 [batch, num_qo_heads, head_dim]) and
 * lse (fp32 [batch, num_qo_heads], may be NULL).  When the two handles' slot
 * counts together fit the compute units (one workgroup each, e.g. half of
 * them each) and the suffix plan runs PKD_VARIANT_MFMA_PV (its default for
 * short suffixes), the two attention kernels are one launch whose
 * workgroups split between the plans, so they run side by side; otherwise
 * they run one after the other.  All launches are on `stream`.  A run
 * captured in a graph replays correctly after re-plans of either handle on
 * the same workspaces (the choice between the two forms is made at the call
 * from the handles' slot counts and the suffix plan's kernel).  Device
 * errors are raised on each handle's own flag.  This is
 * pkd_run_composable_scaled with both scales 1 (which an FP8 E4M3 cache
 * then has). */
int pkd_run_composable(pkd_handle* prefix, pkd_handle* suffix, const void* q, int32_t batch,
                       const void* kv_cache, int64_t num_pages, int32_t q_dtype, int32_t kv_dtype,
                       void* o, float* lse, float sm_scale, pkd_stream_t stream);

/* pkd_run_composable over a cache of FP8 E4M3 codes with one scale per
 * tensor (the meaning of the codes and scales as in pkd_run_scaled): both
 * plans made with kv_dtype PKD_DTYPE_FP8_E4M3.  The same two forms: when
 * the handles' slot counts together fit the compute units, one launch runs
 * the shared-prefix kernel's code on the prefix plan and the FP8 decode
 * kernel's code on the suffix plan side by side; otherwise the two kernels
 * run one after the other; then the same merge.  k_scale and v_scale must
 * be finite and > 0, and 1 for a bf16 cache (else PKD_ERR_INVALID_ARG). */
int pkd_run_composable_scaled(pkd_handle* prefix, pkd_handle* suffix, const void* q,
                              int32_t batch, const void* kv_cache, int64_t num_pages,
                              int32_t q_dtype, int32_t kv_dtype, void* o, float* lse,
                              float sm_scale, float k_scale, float v_scale, pkd_stream_t stream);

/* Waits for `stream`, returns the device error flags raised by runs since
 * the last read (PKD_DEVERR_*, 0 if none) and clears them. */
int pkd_read_device_error(pkd_handle* h, int32_t* flags, pkd_stream_t stream);

/* ------------------------------- append ------------------------------- */

/* The step before decode (pyshine, "The Paged KV Cache Layer"): copy new
 * tokens' K and V rows into their page slots.  All arrays are device arrays.
 *
 * pkd_append_positions: for request i (batch requests), the new tokens
 * append_indptr[i] .. append_indptr[i+1]-1 (int32 [batch+1]) are its last
 * a_i tokens, a_i = append_indptr[i+1] - append_indptr[i]; writes, for each
 * new token, batch_indices[t] = i and positions[t] = L_i - a_i + j, where L_i
 * = page_size (n_i - 1) + kv_last_page_len[i] is the request's length in the
 * page table that already covers the new tokens.
 *
 * pkd_append_paged_kv: new token t (nnz_append of them) with K and V rows
 * k_new[t], v_new[t] (bf16 [nnz_append, num_kv_heads, head_dim], contiguous)
 * goes to request batch_indices[t] at sequence position positions[t], i.e.
 * page kv_indices[kv_indptr[b] + pos / page_size], slot pos % page_size of
 * kv_cache ([num_pages, 2, page_size, num_kv_heads, head_dim], NHD bf16).  A
 * token whose request, position or page id is out of range is not written
 * and sets *device_error (an int32 on the device, may be NULL) to
 * PKD_DEVERR_PAGE_ID.  Only NHD and head_dim 128 are built
 * (PKD_ERR_UNSUPPORTED otherwise); kv_dtype is PKD_DTYPE_BF16 (rows copied
 * bit for bit) or PKD_DTYPE_FP8_E4M3 (rows quantised with scales 1, as
 * pkd_append_paged_kv_scaled).  Asynchronous on `stream`; tokens must not
 * share a slot (the order of such writes is not defined).
 *
 * pkd_append_paged_kv_scaled: pkd_append_paged_kv into an FP8 E4M3 cache
 * with per-tensor scales, quantising as it writes (pyshine, "The Paged KV
 * Cache Layer", on fusing quantisation with the append): a new bf16 value x
 * of K is stored as the E4M3 code nearest to x * (1 / k_scale) (the product
 * in fp32, 1 / k_scale rounded to fp32 once; ties to even; magnitudes above
 * 448 saturate to 448; NaN gives a NaN code), V likewise with v_scale.
 * Scales must be finite and > 0, and 1 with a bf16 cache
 * (PKD_ERR_INVALID_ARG). */
int pkd_append_positions(const int32_t* append_indptr, const int32_t* kv_indptr,
                         const int32_t* kv_last_page_len, int32_t batch, int32_t page_size,
                         int32_t* batch_indices, int32_t* positions, pkd_stream_t stream);
int pkd_append_paged_kv(const void* k_new, const void* v_new, const int32_t* batch_indices,
                        const int32_t* positions, int64_t nnz_append, const int32_t* kv_indptr,
                        const int32_t* kv_indices, int32_t batch, int32_t num_kv_heads,
                        int32_t head_dim, int32_t page_size, int32_t kv_dtype,
                        int32_t kv_layout, void* kv_cache, int64_t num_pages,
                        int32_t* device_error, pkd_stream_t stream);
int pkd_append_paged_kv_scaled(const void* k_new, const void* v_new,
                               const int32_t* batch_indices, const int32_t* positions,
                               int64_t nnz_append, const int32_t* kv_indptr,
                               const int32_t* kv_indices, int32_t batch, int32_t num_kv_heads,
                               int32_t head_dim, int32_t page_size, int32_t kv_dtype,
                               int32_t kv_layout, void* kv_cache, int64_t num_pages,
                               float k_scale, float v_scale, int32_t* device_error,
                               pkd_stream_t stream);

/* -------------------------------- merge ------------------------------- */

/* Merge two attention states row by row: for each of n*H rows,
 * M = max(lse_a, lse_b), w = exp(lse - M), o = (w_a o_a + w_b o_b) / (w_a + w_b),
 * lse = M + log(w_a + w_b) (pinghaoyang page, section on why online softmax
 * allows any split; aicassindra, "Load balancing with split-KV").
 * o_a, o_b, o_out: bf16 [n, H, D]; lse_a, lse_b, lse_out: fp32 [n, H],
 * natural log.  Two empty states (lse = -inf) give o = 0, lse = -inf.
 * o_out / lse_out may alias o_a / lse_a (in-place merge).  Only D = 128. */
int pkd_merge_state(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                    int32_t n, int32_t H, int32_t D, void* o_out, float* lse_out,
                    pkd_stream_t stream);

/* Merge k states per row in index order: o bf16 [n, k, H, D], lse fp32
 * [n, k, H] -> o_out bf16 [n, H, D], lse_out fp32 [n, H].  Only D = 128. */
int pkd_merge_states(const void* o, const float* lse, int32_t n, int32_t k, int32_t H,
                     int32_t D, void* o_out, float* lse_out, pkd_stream_t stream);

/* ------------------------------ profiling ----------------------------- */

/* When enabled, each pkd_run outside graph capture brackets its decode and
 * merge launches with HIP events on its stream; pkd_profile_read waits for
 * them and returns the summed kernel times in milliseconds and the number
 * of runs, then resets the sums.  Off by default. */
int pkd_profile_enable(pkd_handle* h, int32_t enable);
int pkd_profile_read(pkd_handle* h, double* decode_ms, double* merge_ms, int64_t* runs);

/* ------------------------- read-ceiling kernels ----------------------- */

/* Measurement aids, not part of the decode path.  Decode reads every cached
 * key and value once per step, so HBM bandwidth bounds it (aicassindra, "Why
 * serving attention is a different problem"); these kernels only read, and
 * tell how fast this GPU reads with a plain stream and with a page gather,
 * as context for the decode kernels' rate.  Each lane XORs the 32-bit words
 * it reads and writes the result to `sink` (device memory, caller-owned,
 * pkd_read_sink_words(grid) words): the XOR over the sink is the XOR of
 * every word read.  Asynchronous on `stream`; nothing is allocated.
 *
 * pkd_read_stream: `bytes` (a positive multiple of 16) from `buf` (device,
 * 16-byte aligned), each byte once.
 * pkd_read_pages: for each of the n_ids device page ids in order, the whole
 * page of page_bytes (a power of two, at least 16) at base + id * page_bytes;
 * ids outside [0, num_pages) are skipped.  Each workgroup reads a contiguous
 * run of the id list.
 * Both return PKD_ERR_INVALID_ARG on null pointers, bad sizes or alignment,
 * or a grid outside [1, 2^20]. */
int32_t pkd_read_sink_words(int32_t grid);
int pkd_read_stream(const void* buf, int64_t bytes, uint32_t* sink, int32_t grid,
                    pkd_stream_t stream);
int pkd_read_pages(const void* base, int64_t num_pages, int64_t page_bytes,
                   const int32_t* page_ids, int64_t n_ids, uint32_t* sink, int32_t grid,
                   pkd_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKD_H_ */
