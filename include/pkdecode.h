/*
 * pkdecode — batched decode attention over a paged, ragged KV cache on AMD
 * MI355X (gfx950). C ABI.
 *
 * The operation is the paged-KV batch decode of "FlashDecoding + FlashInfer —
 * the decode-time attention story": one query token per request attends over
 * that request's KV tokens, which live in fixed-size pages named by a page
 * table (indptr / indices / last_page_len, §"Paged attention (vLLM) — the
 * KV-cache layout FlashInfer targets"). A request may instead bring a handful
 * of new tokens (speculative or parallel decoding, the page's opening), laid
 * out as ragged q rows by qo_indptr (§"Ragged attention — variable-length
 * batching"); they are the request's last KV tokens and each attends causally
 * (up to and including its own position). Work is split along the KV axis into
 * partial (m, d, o) softmax states that a second kernel merges with the
 * online-softmax rule (§"FlashDecoding — the split-KV trick"), and a host-side
 * plan balances the split so that long requests do not stall short ones
 * (§"What FlashInfer is", item 3). As in the wrapper of §"The API you actually
 * use (Python)", plan() is done once per batch shape on the host and run() is
 * the per-layer hot path.
 *
 * Conventions
 *   - Every function returns PKD_OK (0) or a negative PKD_ERR_* code; the
 *     message of the calling thread's last failure is pkd_last_error().
 *     Nothing aborts the process and no C++ exception crosses this boundary.
 *   - "host" pointers are CPU memory; "device" pointers are HIP device memory
 *     on the plan's device. The caller owns every buffer passed in; the
 *     library allocates only the plan handle (host) and pinned staging blocks
 *     for the work-list copy, which it pools and reuses across plans.
 *   - Streams are hipStream_t passed as void*; NULL is the default stream.
 */
#ifndef PKDECODE_H
#define PKDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define PKD_OK 0
#define PKD_ERR_INVALID_ARGUMENT (-1)   /* malformed page table, null pointer, bad stride */
#define PKD_ERR_UNSUPPORTED (-2)        /* head_dim / group / page_size / dtype not built */
#define PKD_ERR_WORKSPACE_TOO_SMALL (-3)
#define PKD_ERR_PLAN_MISMATCH (-4)      /* run() arguments disagree with the plan */
#define PKD_ERR_HIP (-5)                /* a HIP runtime call failed */

/* ---- element types ----------------------------------------------------- */
#define PKD_DTYPE_F32 0   /* IEEE binary32 */
#define PKD_DTYPE_BF16 1  /* bfloat16 */
#define PKD_DTYPE_E4M3 2  /* OCP FP8 E4M3FN byte, with fp32 per-(page, KV head) scales */
#define PKD_DTYPE_F16 3   /* IEEE binary16 */
/* OCP FP4 E2M1 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit; values
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives), two elements per byte with
 * the lower-indexed one in the low nibble, with fp32 scales per (KV head,
 * channel): the FP4 PageAttention with per-channel scaling factors of
 * "FlashInfer vs FlashAttention-3: GPU Kernel Optimization & FP8 Serving
 * Latency", §"Decision Matrix: Choosing the Right Attention Engine". KV only. */
#define PKD_DTYPE_E2M1 4
/* Signed 4-bit integers in two's complement (codes -8 .. 7), two elements per
 * byte with the lower-indexed one in the low nibble, with fp32 scales per (KV
 * head, channel): value = code x scale. The int4 PageAttention with
 * per-channel scaling factors of the same section of the same page, which
 * gives no encoding; the symmetric two's-complement code is the reading
 * taken. KV only; layout and scales as for PKD_DTYPE_E2M1. */
#define PKD_DTYPE_I4 5

/* Columns of one work item as returned by pkd_plan_get_worklist:
 * request, page_begin, page_end, kv_len, partial_slot, q_row, q_len, visible
 * (see pkd_plan_get_worklist). */
#define PKD_ITEM_COLS 8

typedef struct pkd_plan pkd_plan;

/* Arguments of pkd_plan_create.
 *
 *  batch            number of requests B (>= 1)
 *  indptr           host int32[B+1]: request r owns page-table entries
 *                   [indptr[r], indptr[r+1]); indptr[0] == 0, each request
 *                   has at least one page
 *  last_page_len    host int32[B]: tokens in request r's last page, in
 *                   [1, page_size]; request r holds
 *                   (n_r - 1) * page_size + last_page_len[r] tokens
 *  num_qo_heads     query heads Hq; num_kv_heads divides it and query head h
 *                   reads KV head h / (Hq / Hkv)
 *  head_dim         64 or 128; query heads per KV head 1, 2, 4 or 8, and also
 *                   16 on the MFMA path (head_dim 128: bf16 q over bf16, e4m3,
 *                   e2m1 or int4 KV, fp16 q over fp16 KV) and 32 there except
 *                   for e2m1 and int4 KV
 *  page_size        tokens per page, a power of two in [1, 1024]
 *  q_dtype          PKD_DTYPE_F32, PKD_DTYPE_BF16 or PKD_DTYPE_F16
 *  kv_dtype         PKD_DTYPE_F32, PKD_DTYPE_BF16, PKD_DTYPE_E4M3, PKD_DTYPE_F16
 *                   PKD_DTYPE_E2M1 or PKD_DTYPE_I4; fp16 KV takes fp16 q (and
 *                   fp16 q fp16 KV) at head_dim 128; e2m1 and int4 KV take
 *                   bf16 q at head_dim 128
 *  out_dtype        PKD_DTYPE_F32, PKD_DTYPE_BF16 or PKD_DTYPE_F16 (16-bit
 *                   outputs round to nearest even)
 *  sm_scale         logit scale; 0 selects 1/sqrt(head_dim)
 *  slots            workgroups the device keeps resident at once; 0 queries
 *                   the device (compute units x resident workgroups per CU
 *                   for the selected kernel)
 *  balance          each work unit holds at most 1/balance of a slot's fair
 *                   share of the batch; 0 selects the default (1: one
 *                   round of workgroups; longest-first ordering absorbs the
 *                   raggedness)
 *  min_chunk_pages  shortest chunk a request is split into; 0 selects
 *                   ceil(64 / page_size)
 *  device           HIP device ordinal used when slots == 0
 *  qo_indptr        host int32[B+1] or NULL. NULL: one query token per
 *                   request (q row r). Otherwise request r owns the q rows
 *                   [qo_indptr[r], qo_indptr[r+1]): q_r >= 1 new tokens, at
 *                   most its KV token count, which are its last q_r KV
 *                   tokens in order; new token i attends to the first
 *                   L_r - q_r + 1 + i KV tokens. More than one token per
 *                   request needs head_dim 128 and bf16 q with bf16, e4m3,
 *                   e2m1 or int4 KV, or fp16 q with fp16 KV (else
 *                   UNSUPPORTED); a work item then carries up to 16 / group
 *                   of a request's tokens, or 32 / group (e2m1 and int4:
 *                   16 / group) when a request
 *                   has more (info.queries_per_item).
 *  non_causal       0: the causal rule above. 1: every q row of request r
 *                   sees all of its KV tokens and q_r may exceed them: the
 *                   shared-prefix level of cascade attention, where the
 *                   queries of all requests sharing a prefix attend to it as
 *                   one request (the "Cascade Attention" operator of
 *                   "GitHub Spotlight: FlashInfer", §"Core Superpowers:
 *                   Breaking Down the Feature Set", and its shared-prefix
 *                   use in §"Real-World Deployment Scenarios", Scenario A);
 *                   combine its output with the per-request suffix level
 *                   through pkd_merge_states.
 *  capacity_items,  all 0: the plan is laid out and launched for exactly its
 *  capacity_merge_tasks,  own work list. All > 0: a fixed-capacity plan for
 *  capacity_partials,     HIP graphs. Its workspace layout, launch grids,
 *  capacity_qo_len        kernel choice and kernel arguments depend only on
 *                   these capacities and on the other scalar arguments, not
 *                   on the page table: the kernels read the current counts
 *                   from the workspace and idle workgroups past them return
 *                   at once. A graph that captured pkd_run of one such plan
 *                   therefore computes any other plan with the same scalar
 *                   arguments and capacities once that plan has been
 *                   uploaded to the same workspace (pkd_plan_upload is not
 *                   part of the graph; q, k, v, indices, scales, out and lse
 *                   must be the same buffers, large enough for every plan).
 *                   The plan fails (INVALID_ARGUMENT) if its work items,
 *                   merge tasks (q rows of split requests), partial-state
 *                   rows or most new tokens of one request exceed them.
 *                   Work items never exceed query blocks + slots * balance /
 *                   info.units_per_item (query blocks = B with one token per
 *                   request), and merge tasks and partial rows never exceed
 *                   the q rows and the work items times the tokens per item.
 *  kv_scale_per_token  e4m3 KV only. 0: k_scale/v_scale hold one fp32 scale
 *                   per (page, KV head), [num_pages, Hkv]. 1: one per (token,
 *                   KV head), [num_pages, Hkv, page_size] (a head's scales of a
 *                   page contiguous, 16-byte aligned arrays) — the per-token
 *                   row-wise fp8 scaling of "FlashInfer vs FlashAttention-3:
 *                   GPU Kernel Optimization & FP8 Serving Latency",
 *                   §"Production War Story" (bf16 q and head_dim 128 only).
 *  max_wgs_per_cu   0: the library's default residency for the KV dtype (one
 *                   token per request: one decode workgroup per compute unit,
 *                   two for e2m1 KV, three for int4 KV; several tokens: no
 *                   cap).
 *                   1..4: run() reserves LDS so that at most this many decode
 *                   workgroups share a compute unit (and slots == 0 counts
 *                   them); larger values add no reservation.
 */
typedef struct {
  int32_t batch;
  const int32_t* indptr;
  const int32_t* last_page_len;
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t q_dtype;
  int32_t kv_dtype;
  int32_t out_dtype;
  float sm_scale;
  int32_t slots;
  int32_t balance;
  int32_t min_chunk_pages;
  int32_t device;
  const int32_t* qo_indptr;
  int32_t non_causal;
  int32_t capacity_items;
  int32_t capacity_merge_tasks;
  int32_t capacity_partials;
  int32_t capacity_qo_len;
  int32_t max_wgs_per_cu;
  int32_t kv_scale_per_token;
} pkd_plan_args;

/* What a plan decided (pkd_plan_get_info). */
typedef struct {
  int32_t batch;
  int32_t chunk_pages;         /* C: pages per work item (the last chunk may be shorter) */
  int32_t num_items;           /* work items; the decode grid is num_items x num_kv_heads */
  int32_t num_partials;        /* partial-state rows (per q row of each chunk of split requests) */
  int32_t num_split_requests;  /* requests with more than one item */
  int32_t slots;               /* values actually used by the rule */
  int32_t balance;
  int32_t min_chunk_pages;
  int64_t total_kv_tokens;     /* sum over requests of their token counts */
  size_t workspace_bytes;      /* device workspace run() needs */
  int32_t query_rows;          /* rows of q, out and lse (B with one token per request) */
  int32_t queries_per_item;    /* new tokens of one request a work item carries at most */
  int32_t max_qo_len;          /* most new tokens of one request */
  int32_t num_merge_tasks;     /* q rows of split requests (merge grid / num_qo_heads) */
  int32_t units_per_item;      /* decode workgroups per work item: one per KV head or
                                  per pair of KV heads */
  int32_t merge_folded;        /* 1: pkd_run folds the merge into the decode kernel */
  int32_t slots_per_cu;        /* resident workgroups per compute unit the rule took
                                  (the device query's; 1 when slots was given) */
} pkd_plan_info;

/* Arguments of pkd_run. All pointers are device pointers.
 *
 *  q            [rows, Hq, head_dim] contiguous, q_dtype (rows =
 *               info.query_rows: B, or qo_indptr[B])
 *  k, v         element (page 0, slot 0, KV head 0, dim 0) of the K and V
 *               pools; element (page, slot, h, d) of K is at
 *               k[page*page_stride + slot*token_stride + h*head_stride + d]
 *               (same for v). The combined NHD pool
 *               [num_pages, 2, page_size, Hkv, head_dim] is
 *               k = base, v = base + page_size*Hkv*head_dim,
 *               page_stride = 2*page_size*Hkv*head_dim,
 *               token_stride = Hkv*head_dim, head_stride = head_dim.
 *               Strides are in elements (e2m1 and int4: two per byte, so the
 *               combined pool's strides above hold with head_dim counted in
 *               elements); k, v and every stride must be 16-byte aligned for
 *               f32/bf16/f16/e2m1/int4 and 8-byte aligned for e4m3, and a
 *               page (page_stride) must span less than 4 GiB.
 *  indices      int32 page ids of the page table (length indptr[B]); ids may
 *               repeat across requests (shared prefixes) and are not range
 *               checked (pkd_check_page_ids does that off the hot path)
 *  k_scale,     e4m3: float [num_pages, Hkv] contiguous (or, with
 *  v_scale      kv_scale_per_token, [num_pages, Hkv, page_size]): stored K
 *               (V) bytes are multiplied by the scale of their (page, KV
 *               head) or (token, KV head). e2m1 and int4: float [Hkv, head_dim]
 *               contiguous, element (h, d) multiplying channel d of every
 *               K (V) row of KV head h. Required for e4m3, e2m1 and int4 KV,
 *               ignored otherwise; row-wise and per-channel arrays must be
 *               16-byte aligned.
 *  out          [rows, Hq, head_dim] contiguous, out_dtype
 *  lse          float [rows, Hq] or NULL: natural-log log-sum-exp of the
 *               scaled logits of each (q row, query head)
 *  workspace    the buffer the plan was uploaded to, at least
 *               info.workspace_bytes long
 *  stream       hipStream_t; run() only enqueues work and returns
 *  prior_out,   NULL, or another normalised result of the same q rows over a
 *  prior_lse    disjoint token set (the other level of cascade attention):
 *               float [rows, Hq, head_dim] and its natural-log LSE float
 *               [rows, Hq] (-inf: a result over no tokens), both contiguous,
 *               16-byte aligned, not aliasing out or lse. run() then writes
 *               the merge of its own result with it, by the rule of
 *               pkd_merge_states, to out and lse (both sides empty: 0 and
 *               -inf), in place of a separate merge launch. Both or neither.
 */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  int64_t page_stride;
  int64_t token_stride;
  int64_t head_stride;
  const int32_t* indices;
  const float* k_scale;
  const float* v_scale;
  void* out;
  float* lse;
  void* workspace;
  size_t workspace_bytes;
  void* stream;
  const float* prior_out;
  const float* prior_lse;
} pkd_run_args;

/* Message describing the calling thread's most recent failure ("" if none). */
const char* pkd_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int pkd_version(void);

/* Validate the page table and build the work partition on the host.
 * Rejects empty requests, last_page_len outside [1, page_size], a
 * non-monotone indptr, Hq not a multiple of Hkv (INVALID_ARGUMENT) and
 * head_dim / group / page_size / dtype combinations with no kernel
 * (UNSUPPORTED). On success *out owns a new handle. No device work. */
int pkd_plan_create(const pkd_plan_args* args, pkd_plan** out);

/* Copy out what the plan decided. */
int pkd_plan_get_info(const pkd_plan* plan, pkd_plan_info* info);

/* Copy the work list to host memory: items_out int32[num_items * 8] rows of
 * (request, page_begin, page_end, kv_len, partial_slot, q_row, q_len,
 * visible) in launch order. An item covers page-table entries
 * [page_begin, page_end) (kv_len tokens) for the q_len q rows from q_row;
 * the first of those rows sees min(kv_len, visible) of the item's tokens and
 * row i sees min(kv_len, visible + i) (kv_len itself with one token per
 * request). partial_slot is -1 for a request that is not split, else the
 * partial-state row of q row q_row (row i uses partial_slot + i).
 * merge_indptr_out int32[B+1]: the split request r owns partial-state rows
 * [merge_indptr[r], merge_indptr[r+1]), chunk c's row for its token i being
 * merge_indptr[r] + c * q_r + i; split_requests_out (nullable)
 * int32[num_split_requests], the split requests in ascending order. */
int pkd_plan_get_worklist(const pkd_plan* plan, int32_t* items_out, int32_t* merge_indptr_out,
                          int32_t* split_requests_out);

/* Enqueue the copy of the work list into the head of `workspace` on
 * `stream` (asynchronous; the plan keeps its pinned staging copy alive
 * until the copy has finished). run() must then be given the same workspace. */
int pkd_plan_upload(pkd_plan* plan, void* workspace, size_t workspace_bytes, void* stream);

/* Enqueue the run on args->stream: the decode kernel and, when a request was
 * split, the merge. For an exact plan whose split requests have at most
 * sixteen chunks, with at most 64 workgroups working on split requests in all, the
 * merge is folded into the decode kernel (one launch): the last
 * workgroup of each split request (per query block and KV head) folds its
 * partial states into the output rows, counting chunk arrivals with an
 * atomic counter kept in the workspace, which it leaves at zero. Otherwise
 * (longer folds, fixed-capacity plans) the separate merge kernel follows.
 * Allocates nothing and does not synchronise. */
int pkd_run(const pkd_plan* plan, const pkd_run_args* args);

/* Stages of run(), kept apart, for callers that time or interleave them or
 * combine partial states themselves: the split-KV decode kernel alone
 * (partial states of split requests, final rows of the others) and the
 * separate merge kernel that folds the partial states (a no-op when none is
 * split). PKD_STAGE_ALL is pkd_run. The merge stage reads what the decode
 * stage of the same plan and workspace wrote. */
#define PKD_STAGE_DECODE 1
#define PKD_STAGE_MERGE 2
#define PKD_STAGE_ALL 3
int pkd_run_stages(const pkd_plan* plan, const pkd_run_args* args, int32_t stages);

/* pkd_run_stages, with the decode kernel's own dispatch recording two HIP
 * events: `decode_start` when the kernel begins executing and `decode_stop`
 * when it has completed (hipExtLaunchKernel's kernel events), so that
 * hipEventElapsedTime between them is the kernel's duration without the
 * queue's packet overhead that events recorded around the launch include.
 * Both are hipEvent_t passed as void*, created on the plan's device with
 * timing enabled and owned by the caller; either may be NULL (then it is
 * not recorded). They are ignored when `stages` does not include
 * PKD_STAGE_DECODE. For callers that measure the decode kernel; the work
 * enqueued is that of pkd_run_stages. */
int pkd_run_timed(const pkd_plan* plan, const pkd_run_args* args, int32_t stages,
                  void* decode_start, void* decode_stop);

/* pkd_run for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops and harnesses that forbid allocation): the same
 * kernels and results as pkd_run, but the plan's work list, merge records,
 * fold counters and partial states live in a scratch array the library holds
 * in each device's memory (16 MiB, a static device array, from the library's
 * load until the process ends) instead of a caller-allocated workspace;
 * args->workspace and args->workspace_bytes are ignored and the plan needs no
 * pkd_plan_upload. The call enqueues on args->stream a copy of the plan's
 * work list (from the plan's host image, which it has read when it returns)
 * into the current device's scratch, then the run, and allocates nothing.
 * A plan whose info.workspace_bytes exceeds the scratch is refused with
 * PKD_ERR_WORKSPACE_TOO_SMALL. Every call on a device uses that device's one
 * scratch array: calls that may overlap on one device (other streams, other
 * threads) race and must be ordered by the caller. */
int pkd_run_static(const pkd_plan* plan, const pkd_run_args* args);

/* Count the page ids among indices[0 .. count) (device memory) that lie
 * outside [0, num_pages), the pool's page count, after the work already
 * queued on `stream`: the call copies the ids to the host and synchronises
 * the stream. *bad_out receives the count and *first_bad_out (may be NULL)
 * the position of the first such id, or -1. run() does not range-check
 * page ids (they are read on the hot path, per tile), and an id outside the
 * pool makes the decode kernel read outside it; this is the check for
 * callers that validate a page table once before using it (the Python
 * wrapper runs it before run() when asked to). Allocates host memory only. */
int pkd_check_page_ids(const int32_t* indices, int64_t count, int32_t num_pages, void* stream,
                       int64_t* bad_out, int64_t* first_bad_out);

/* Free the handle. Its pinned staging block returns to a process-wide pool
 * and is handed to another plan only after its last copy has completed, so
 * destroying a plan never waits. NULL is a no-op. */
void pkd_plan_destroy(pkd_plan* plan);

/* Arguments of pkd_merge_states. Device pointers.
 *
 *  rows, num_heads, head_dim   shape [rows, num_heads, head_dim] of v_a, v_b
 *                              and v_out; head_dim a multiple of 4
 *  in_dtype                    PKD_DTYPE_F32, PKD_DTYPE_BF16 or PKD_DTYPE_F16 (v_a, v_b)
 *  out_dtype                   PKD_DTYPE_F32, PKD_DTYPE_BF16 or PKD_DTYPE_F16 (v_out)
 *  v_a, s_a, v_b, s_b          two normalised attention results over disjoint
 *                              token sets: output rows and their natural-log
 *                              log-sum-exp, float [rows, num_heads];
 *                              s = -inf marks a result over no tokens
 *  v_out, s_out                merged result; s_out may be NULL; v_out may
 *                              alias v_a or v_b when the dtypes agree, s_out
 *                              may alias s_a or s_b
 *  stream                      hipStream_t
 *
 * Pointers to f32 rows must be 16-byte aligned, to 16-bit rows 8-byte aligned. */
typedef struct {
  int64_t rows;
  int32_t num_heads;
  int32_t head_dim;
  int32_t in_dtype;
  int32_t out_dtype;
  const void* v_a;
  const float* s_a;
  const void* v_b;
  const float* s_b;
  void* v_out;
  float* s_out;
  void* stream;
} pkd_merge_states_args;

/* Merge two normalised results of the same queries over disjoint token sets
 * with the online-softmax rule of "FlashDecoding + FlashInfer — the
 * decode-time attention story", §"FlashDecoding — the split-KV trick": a
 * result (v, s) is the state (m = s, d = 1, o = v), so
 *   s_out = max(s_a, s_b) + ln(w_a + w_b),  w_x = exp(s_x - max(s_a, s_b)),
 *   v_out = (w_a v_a + w_b v_b) / (w_a + w_b).
 * Both sides empty gives v_out = 0, s_out = -inf. Enqueues one kernel. */
int pkd_merge_states(const pkd_merge_states_args* args);

/* Workgroups of the decode kernel selected for (q_dtype, kv_dtype, head_dim,
 * group, page_size) and one query token per request that one compute unit
 * holds at once, and the device's compute-unit count. On the MFMA path with
 * an even number of KV heads and pages of at least 16 tokens one workgroup
 * serves a pair of KV heads (info.units_per_item of a plan gives the
 * workgroups per work item). */
int pkd_device_slots(int32_t device, int32_t q_dtype, int32_t kv_dtype, int32_t head_dim,
                     int32_t group, int32_t page_size, int32_t* wgs_per_cu, int32_t* num_cus);

/* Calibration: enqueue one plain streaming read of `bytes` bytes at `buf`
 * (device memory, 16-byte aligned, bytes a positive multiple of 16) by
 * `workgroups` workgroups of four wavefronts, each keeping 8 KiB per
 * wavefront in flight over consecutive 32 KiB blocks, with non-temporal
 * loads (the data is read once). `sink` (device,
 * uint32[4 * workgroups]) receives an XOR of the data so that the reads are
 * not optimised away. Timing it (events on `stream`) gives the HBM read rate
 * one kernel reaches on the device, the ceiling the decode kernels' KV-read
 * rate is set against: the pages measure decode kernels as a fraction of
 * memory bandwidth ("Attention Kernel Comparison: FlashAttention vs
 * FlashInfer vs xformers vs Triton", opening paragraphs). */
int pkd_stream_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKDECODE_H */
