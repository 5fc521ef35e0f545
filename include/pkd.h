/*
 * pkd.h - paged-KV batch decode attention on AMD MI355X (gfx950, CDNA4).
 *
 * The operation is the one of flashinfer.decode.BatchDecodeWithPagedKVCacheWrapper
 * on the "FlashInfer attention kernels" API page: every request of a batch has
 * ONE query token per q head, and it attends the keys/values stored in that
 * request's pages of a paged KV cache. Pages are found through a CSR page
 * table (indptr / indices / last_page_len). q heads are grouped onto kv heads
 * (grouped-query attention). Options: sm_scale, logits_soft_cap, window_left,
 * fixed_split_size / disable_split_kv, fp8 E4M3 keys/values with calibration
 * scales. A long sequence may be cut into chunks whose partial states are
 * combined by a log-sum-exp merge (the merge_states step named on that page).
 *
 * Definitions used throughout (same page and section):
 *   B        batch size; request i owns pages indices[indptr[i] .. indptr[i+1])
 *   P        page_size; 1 <= last_page_len[i] <= P (class example comment)
 *   L_i      kv_len = P*(indptr[i+1]-indptr[i]-1) + last_page_len[i]
 *            (kv_len expression of the prefill wrapper's custom-mask example)
 *   G        num_qo_heads / num_kv_heads; q head hq reads kv head hq / G
 *   window   window_left >= 0 keeps tokens t >= L_i-1-window_left (inclusive
 *            left window; the query sits at position L_i-1); -1 keeps all
 *   logits   x = sm_scale*q_scale*k_scale * (q . k); if logits_soft_cap > 0,
 *            x <- cap*tanh(x/cap)
 *   o        sum_t softmax(x)_t * v_scale * v_t ;  lse = ln sum_t exp(x_t)
 *   Q        q_len_per_req (run() parameter of the same wrapper, default 1):
 *            query tokens per request. q, o and lse then hold Q consecutive
 *            rows per request, in token order; query token j sits at
 *            position L_i-Q+j (the causal diagonal kv_len-qo_len of the
 *            prefill wrapper's mask example) and attends t <= L_i-Q+j, and
 *            with a window also t >= L_i-Q+j-window_left
 *
 * Memory and streams.
 *   Every device buffer (q, caches, indices, o, lse, workspace) is owned by
 *   the caller. `stream` arguments are hipStream_t values passed as void*
 *   (NULL = the default stream). pkd_run* only enqueue work on `stream`: they
 *   never allocate, never synchronise and never read device memory on the
 *   host.
 *
 * Errors.
 *   Every call returns a pkd_status; on failure pkd_last_error() returns a
 *   thread-local message that names the offending value and the limit.
 *   Nothing is launched when a call fails.
 */
#ifndef PKD_H_
#define PKD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKD_ABI_VERSION 4

typedef enum {
  PKD_OK = 0,
  PKD_EINVAL = -1,        /* invalid argument or page table               */
  PKD_EUNSUPPORTED = -2,  /* valid, but not built (head_dim, dtype, ...)  */
  PKD_EHIP = -3,          /* a HIP runtime call failed                    */
  PKD_ENOMEM = -4,        /* host or device allocation failed (plan only) */
  PKD_EWORKSPACE = -5     /* workspace missing or smaller than required   */
} pkd_status;

/* Stored element types. E4M3 is the OCP fp8 "fn" format (torch.float8_e4m3fn):
 * bias 7, no infinities, NaN = 0x7F/0xFF, largest finite 448. */
typedef enum { PKD_F16 = 0, PKD_BF16 = 1, PKD_E4M3 = 2, PKD_F32 = 3 } pkd_dtype;

/* Cache layouts of the run() parameter paged_kv_cache:
 *   NHD: one page of K (or V) is [P][num_kv_heads][head_dim]
 *   HND: one page of K (or V) is [num_kv_heads][P][head_dim]
 * head_dim is always contiguous. */
typedef enum { PKD_NHD = 0, PKD_HND = 1 } pkd_layout;

/* Positional encoding applied inside the kernel (plan() parameter
 * pos_encoding_mode). ALIBI adds slope_h * (t - p) to the scaled logit of q
 * head h for key position t and query position p, before the soft cap; the
 * slopes are those of the ALiBi paper over num_qo_heads heads: with
 * n = 2^floor(log2 num_qo_heads), head h < n gets 2^(-8(h+1)/n), head
 * h >= n gets 2^(-4(2(h-n)+1)/n). */
typedef enum { PKD_POS_NONE = 0, PKD_POS_ROPE_LLAMA = 1, PKD_POS_ALIBI = 2 } pkd_pos_encoding;

/* Problem description of plan(). Enum-valued fields are int32_t (values from
 * the enums above) so that the struct layout is fixed. */
typedef struct {
  int32_t batch_size;       /* B >= 0                                       */
  int32_t num_qo_heads;     /* >= 1, a multiple of num_kv_heads             */
  int32_t num_kv_heads;     /* >= 1; G = num_qo_heads/num_kv_heads, any    */
  int32_t head_dim;         /* 64, 128 or 256                               */
  int32_t page_size;        /* a power of two, 1 .. 256                     */
  int32_t layout;           /* pkd_layout                                   */
  int32_t q_dtype;          /* PKD_F16 or PKD_BF16                          */
  int32_t kv_dtype;         /* q_dtype or PKD_E4M3                          */
  int32_t o_dtype;          /* PKD_F16 or PKD_BF16                          */
  float sm_scale;           /* finite; 1/sqrt(head_dim) is the usual value  */
  float logits_soft_cap;    /* <= 0: off; else cap*tanh(x/cap)              */
  int32_t window_left;      /* -1: whole sequence; >= 0: inclusive window   */
  int32_t fixed_split_size; /* pages per chunk; 0: the planner chooses      */
  int32_t disable_split_kv; /* nonzero: exactly one chunk per request       */
  int32_t q_len_per_req;    /* Q, query tokens per request; 0 means 1;
                               Q <= 16 and every L_i >= Q                   */
  int32_t pos_encoding_mode; /* pkd_pos_encoding. ROPE_LLAMA turns q at its
                               position L_i - Q + j and each key at its token
                               index (pairs d, d + head_dim/2); it is
                               PKD_EUNSUPPORTED for kv lengths above 2^24  */
  float rope_scale;         /* ROPE_LLAMA: angle = pos / rope_scale *       */
  float rope_theta;         /* rope_theta^(-2d/head_dim); both positive and
                               finite (else PKD_EINVAL), unused otherwise   */
} pkd_plan_params;

/* One unit of decode work: the tokens [token_begin, token_end) of one chunk of
 * one request, for one kv head and its G q heads, or a block of them (below),
 * and the Q query tokens.
 * Tokens past a query token's position, or before its window, are masked
 * for that token only. Under a fixed split, chunks
 * longer than 3072 tokens are processed as units of 3072 tokens cut at fixed
 * offsets from the chunk start, so each unit depends on its request alone.
 * Under the planner's own split a request is cut into units of equal length
 * (to the token, the cuts then moved to multiples of 32 tokens unless a unit
 * would pass the cap), as few as keep each within split_pages pages; a batch
 * too small to give every workgroup 256 tokens is cut as a fixed split of
 * split_pages would cut it.
 * A unit carries at most 16 query rows (G*Q). A larger group is split into
 * the fewest nb equal blocks of G/nb q heads with (G/nb)*Q <= 16, and
 * kv_head then numbers blocks: block b of kv head h is kv_head h*nb + b, it
 * covers q heads (h*nb + b)*(G/nb) .. + G/nb - 1 and reads kv head h's K/V
 * (each block reads it once; a group with no divisor that fits runs one q
 * head per block). */
typedef struct {
  int32_t request;
  int32_t kv_head;
  int32_t token_begin;      /* first attended token of the chunk            */
  int32_t token_end;        /* one past the last attended token             */
  int32_t page_base;        /* indptr[request] (block table: request*row)   */
  int32_t partial;          /* -1: writes o/lse; else its workspace slot    */
  int32_t chunk;            /* unit index within the request (ascending)    */
  int32_t num_chunks;       /* units of the request per kv_head (1: unsplit) */
  int32_t query_pos;        /* position of the request's first query token,
                               L_i - Q                                      */
} pkd_work_item;

typedef struct {
  int32_t num_items;        /* work items (units of decode work)            */
  int32_t num_workgroups;   /* decode workgroups; they take items in order  */
  int32_t num_split_requests; /* requests cut into more than one unit       */
  int32_t num_partials;     /* workspace slots (units of split requests)    */
  int32_t split_pages;      /* fixed split: chunk size in pages; planner's
                               split: longest unit in pages; 0 = no split   */
  int32_t workgroups_per_cu; /* decode workgroups resident per compute unit */
  int64_t attended_tokens;  /* sum over requests of attended tokens         */
  size_t workspace_bytes;   /* bytes the workspace of pkd_run must hold     */
} pkd_plan_info;

typedef struct pkd_plan pkd_plan; /* opaque, owned by the library */

/* Library housekeeping (no passage of the page): PKD_ABI_VERSION of the
 * built library, for a binding to check against this header. */
int32_t pkd_abi_version(void);

/* Library housekeeping (no passage; the page's wrappers raise exceptions
 * that name the violated limit, which this message carries to a binding):
 * message of the last failed call on this thread ("" if none). The pointer
 * stays valid until the next pkd_* call on the same thread. */
const char* pkd_last_error(void);

/* plan(): validate the page table, choose the chunking and build the work
 * list (flashinfer.decode › BatchDecodeWithPagedKVCacheWrapper › plan()).
 *   indptr         host, int32 [B+1], read during the call only
 *   last_page_len  host, int32 [B],   read during the call only
 *   indices        DEVICE, int32 [indptr[B]], BORROWED: it must stay alive and
 *                  unchanged while the plan is used; every entry must index a
 *                  page of the caches given to pkd_run (not checked on device)
 *   stream         the work list is uploaded with an asynchronous copy on it
 * On success *out owns device memory and pinned host memory until
 * pkd_plan_destroy. Not capturable in a HIP graph (it allocates). Errors:
 * PKD_EINVAL (page table or parameter out of range, null pointer),
 * PKD_EUNSUPPORTED (head_dim, G, page_size or dtype combination not built),
 * PKD_ENOMEM / PKD_EHIP. */
pkd_status pkd_plan_create(const pkd_plan_params* params, const int32_t* indptr,
                           const int32_t* last_page_len, const int32_t* indices,
                           void* stream, pkd_plan** out);

/* Host-only planning: the same validation and chunking as pkd_plan_create for
 * a gfx950 GPU with `num_cus` compute units (the number of decode workgroups
 * per compute unit is taken from the library's build), without any HIP call.
 * Writes *info and, if items != NULL, up to `capacity` work items in the
 * order the decode workgroups take them (longest first). */
pkd_status pkd_plan_query(const pkd_plan_params* params, const int32_t* indptr,
                          const int32_t* last_page_len, int32_t num_cus,
                          pkd_plan_info* info, pkd_work_item* items,
                          int32_t capacity);

/* plan() from a block table instead of the CSR page table: the page_table /
 * seq_lens input of the XQA decode on the same page ("page_table" [batch,
 * nb_pages_per_seq] int32, K and V sharing it; "seq_lens" per request), also
 * the seq_lens / block_tables parameters of the trtllm-gen prefill plan().
 *   seq_lens       host, int32 [B], L_i >= 1 (>= Q), read during the call only
 *   block_tables   DEVICE, int32 [B][max_blocks_per_seq], row-major,
 *                  BORROWED like indices: request i owns pages
 *                  block_tables[i][0 .. ceil(L_i/P)); later entries of the
 *                  row are never read
 * Equivalent to pkd_plan_create with indptr[i+1]-indptr[i] = ceil(L_i/P),
 * last_page_len[i] = L_i - P*(ceil(L_i/P)-1) and the index array read at
 * row i of the table; runs of such a plan give the same bits as that plan.
 * Errors as pkd_plan_create, and PKD_EINVAL when max_blocks_per_seq < 1 or
 * a request needs more pages than a row holds. */
pkd_status pkd_plan_create_block_table(const pkd_plan_params* params, const int32_t* seq_lens,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       void* stream, pkd_plan** out);

/* Host-only planning of a block-table batch (as pkd_plan_query). The
 * items' page_base is i * max_blocks_per_seq. */
pkd_status pkd_plan_query_block_table(const pkd_plan_params* params, const int32_t* seq_lens,
                                      int32_t max_blocks_per_seq, int32_t num_cus,
                                      pkd_plan_info* info, pkd_work_item* items,
                                      int32_t capacity);

/* A graph plan: the CUDAGraph-compatible decode wrapper of the same page
 * (CUDAGraphBatchDecodeWithPagedKVCacheWrapper: fixed indptr / indices /
 * last_page_len buffers, a batch size fixed for the wrapper's life, plan()
 * not capturable). Such a plan keeps its device memory, its launch size (one
 * workgroup per slot of the GPU; those without a unit exit at once) and its
 * workspace layout for its whole life, sized for any page table of
 * params->batch_size requests holding at most max_pages pages, so that a
 * pkd_run recorded once in a HIP graph serves every later
 * pkd_plan_update. The kernel reads the current unit count from the plan's
 * device memory.
 *   max_pages   capacity of `indices` (entries), >= indptr[B]
 *   indices     DEVICE, BORROWED for the plan's life; the caller writes each
 *               page table's page ids into it before (stream order) the
 *               runs that use them
 * pkd_plan_info.workspace_bytes is then the capacity's (the same after every
 * update). Errors as pkd_plan_create, and PKD_EINVAL for batch_size < 1,
 * max_pages < 1 or a page table with more pages; PKD_EUNSUPPORTED when the
 * capacity exceeds the 2 GiB workspace or the 2^24 unit limits. */
pkd_status pkd_plan_create_graph(const pkd_plan_params* params, int32_t max_pages,
                                 const int32_t* indptr, const int32_t* last_page_len,
                                 const int32_t* indices, void* stream, pkd_plan** out);

/* A new page table for a graph plan (same parameters and batch size):
 * plans it on the host, waits for the plan's previous upload, and uploads
 * the new work list on `stream` into the same device memory, ordered (on
 * the GPU) after the plan's last tracked run. Runs of the plan must be
 * stream-ordered after it, and replays of graphs holding its runs must not
 * be in flight. Not capturable. Errors: PKD_EINVAL (not a graph plan, NULL,
 * more than max_pages pages, invalid page table), PKD_EUNSUPPORTED (more
 * units than the capacity; not expected within max_pages), PKD_EHIP. On
 * error the plan keeps its previous page table. */
pkd_status pkd_plan_update(pkd_plan* plan, const int32_t* indptr,
                           const int32_t* last_page_len, void* stream);

/* Size of the workspace pkd_run needs for this plan, in bytes (0 when no
 * request is split). The decode wrapper's constructor takes the workspace
 * from the caller (float_workspace_buffer, the buffer that holds split-KV
 * partial states); this is how a caller sizes it. Errors: PKD_EINVAL for
 * a NULL argument. */
pkd_status pkd_plan_workspace_bytes(const pkd_plan* plan, size_t* bytes);

/* What plan() decided (the chunking of fixed_split_size / disable_split_kv
 * and the planner's own split of the same plan() section), for callers and
 * tests: unit and workgroup counts, split size, attended tokens, workspace
 * bytes. Errors: PKD_EINVAL for a NULL argument. */
pkd_status pkd_plan_get_info(const pkd_plan* plan, pkd_plan_info* info);

/* Library housekeeping (no passage; the counterpart of the wrapper object
 * going away): waits for the plan's upload to finish, then frees it. The
 * caller must not destroy a plan whose runs are still in flight. NULL is a
 * no-op. */
void pkd_plan_destroy(pkd_plan* plan);

/* run() (flashinfer.decode › BatchDecodeWithPagedKVCacheWrapper › run()):
 *   q        device, [B*Q][num_qo_heads][head_dim] in q_dtype, contiguous
 *   k_cache  device, K pages in kv_dtype and the plan's layout
 *   v_cache  device, V pages; for the 5-D cache [pages][2][...] pass
 *            v_cache = k_cache + P*num_kv_heads*head_dim elements
 *   page_stride  elements from one page to the next in k_cache and v_cache:
 *            2*P*num_kv_heads*head_dim for the 5-D cache,
 *            P*num_kv_heads*head_dim for a (k_cache, v_cache) pair
 *   q_scale, k_scale, v_scale  calibration scales (1.0 = none)
 *   sinks    device fp32 [num_qo_heads] (the XQA decode's "sinks"
 *            [num_kv_heads][G], flattened in q-head order), or NULL: the
 *            sink s of a q head is one more logit of its softmax, in the
 *            units of the final logits x and never capped, with no value
 *            row: o = sum_t e^x_t v_t / (sum_t e^x_t + e^s) and
 *            lse = ln(sum_t e^x_t + e^s); -inf is no sink
 *   o        device, [B*Q][num_qo_heads][head_dim] in o_dtype, written
 *   lse      device, [B*Q][num_qo_heads] fp32 natural-log LSE, or NULL
 *   workspace, workspace_bytes  device scratch of at least
 *            pkd_plan_info.workspace_bytes (may be NULL when that is 0); its
 *            contents need no initialisation
 * One kernel launch. Units of a split request write partial states to the
 * workspace; the workgroup that finishes the last unit of a (request, kv
 * head) merges that request's partials for the head by log-sum-exp in
 * ascending chunk order (merge_states named with fixed_split_size), so the
 * result does not depend on which workgroup ran which unit.
 * Workgroups that run out of units may take a long unit another workgroup
 * holds in reserve; which workgroup runs a unit never changes the result.
 * Runs of one plan never overlap in time: the workgroups share work
 * counters, reserve slots and merge counters owned by the plan, so a run
 * on a stream other than that of the plan's previous run first waits, on
 * the GPU, for that run (an event the library records after each run; no
 * host synchronisation). Runs of different plans may overlap. Runs
 * recorded into a HIP graph, and their replays, are not tracked: a graph's
 * runs of one plan must be ordered by the caller.
 * Alignment: q, k_cache, v_cache 16 bytes (and page_stride a multiple of 16
 * bytes), o 8 bytes, workspace 256 bytes.
 * The stream must be on the plan's device (the current device for NULL).
 * Errors: PKD_EINVAL (null pointer, page_stride too small, misaligned
 * buffer, a stream of another device), PKD_EWORKSPACE, PKD_EHIP (launch
 * failure). */
pkd_status pkd_run(const pkd_plan* plan, const void* q, const void* k_cache,
                   const void* v_cache, int64_t page_stride, float q_scale,
                   float k_scale, float v_scale, const float* sinks, void* o,
                   float* lse, void* workspace, size_t workspace_bytes,
                   void* stream);

/* pkd_run without a workspace argument, for callers that cannot allocate
 * one: code being captured into a HIP graph, tight serving loops, harnesses
 * that forbid device allocation. The split-KV partial states go to a static
 * workspace the library holds on each GPU it runs on (PKD_STATIC_WORKSPACE_BYTES,
 * 32 MiB, kept until the process ends); this call allocates nothing and
 * computes exactly what pkd_run computes with the same plan (the same
 * kernel and bits). The workspace needs no clearing: every partial state is
 * written before it is read, and the counters are the plan's.
 * All calls on one GPU share that GPU's static workspace, for any plan, so
 * a call on a stream other than that of the previous such call on the GPU
 * first waits, on the GPU, for it (as runs of one plan do). Calls recorded
 * into a HIP graph, and their replays, are not tracked: they race with any
 * other use of the static workspace that overlaps them. The current device
 * must be the plan's.
 * Arguments as pkd_run. Errors: as pkd_run, and PKD_EWORKSPACE when the
 * plan needs more than PKD_STATIC_WORKSPACE_BYTES (pkd_plan_workspace_bytes
 * tells beforehand), PKD_EINVAL when the current device is not the plan's,
 * PKD_EHIP when the static workspace's address is unavailable. */
#define PKD_STATIC_WORKSPACE_BYTES ((size_t)32 << 20)
pkd_status pkd_run_static_workspace(const pkd_plan* plan, const void* q, const void* k_cache,
                                    const void* v_cache, int64_t page_stride, float q_scale,
                                    float k_scale, float v_scale, const float* sinks,
                                    void* o, float* lse, void* stream);

/* merge_states (named with fixed_split_size in plan()): combine `num_states`
 * attention states per row by log-sum-exp:
 *   M = max_k s[k];  Z = sum_k exp(s[k] - M);  s_out = M + ln Z;
 *   v_out = sum_k exp(s[k] - s_out) * v[k]
 * The summation order depends only on num_states (deterministic).
 *   v      device fp32 [rows][num_states][head_dim], per-state normalised o
 *   s      device fp32 [rows][num_states], per-state natural-log LSE;
 *          -inf marks an empty state, which contributes nothing
 *   v_out  device [rows][head_dim] in out_dtype (F16, BF16 or F32)
 *   s_out  device fp32 [rows] natural-log LSE, or NULL
 * A row whose states are all empty gets v_out = 0 and s_out = -inf.
 * head_dim is 1 .. 1024. Errors: PKD_EINVAL, PKD_EUNSUPPORTED, PKD_EHIP. */
pkd_status pkd_merge_states(const float* v, const float* s, int32_t rows,
                            int32_t num_states, int32_t head_dim, void* v_out,
                            int32_t out_dtype, float* s_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKD_H_ */
