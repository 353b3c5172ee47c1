/*
 * pkv — single-token paged attention decode for AMD MI355X (gfx950).
 *
 * C ABI of the library libpkv.so. Every entry point returns a pkv_status
 * (PKV_OK == 0); on failure pkv_last_error() gives a thread-local message.
 * No entry point allocates device memory or synchronises: run, merge and
 * gather only enqueue kernels on the caller's HIP stream. The caller owns every
 * device buffer (inputs, outputs, workspace); the library owns only the host
 * plan object.
 *
 * What is computed (paged GQA decode; kernelindex.com, "flashinfer
 * gemini-2.5-pro / triton h7ykt0", kernel gqa_paged_decode_h32_kv4_d128_ps1,
 * steps 2-9, and its wrapper run()): for sequence b with n = indptr[b+1] -
 * indptr[b] tokens, token j stored in page p_j = kv_indices[kv_indptr[b] + j],
 * and query head h reading KV head g = h / (Hq / Hkv):
 *
 *     s_j      = sm_scale * dot(q[b,h,:], K[p_j, 0, g, :])
 *     out[b,h] = sum_j exp(s_j) V[p_j, 0, g, :] / sum_j exp(s_j)   (bf16)
 *     lse[b,h] = log2(sum_j exp(s_j))                               (fp32)
 *
 * and out = 0, lse = -inf when n == 0. Long sequences are split into chunks
 * whose normalised fp32 partials and base-2 LSEs are combined by pkv_merge
 * (vLLM fork qsa.py, _qsa_sparse_paged_gqa_splitk_kernel and
 * _qsa_merge_splitk_kernel).
 *
 * Supported shapes (compiled in): Hq = 32, Hkv = 4, head_dim = 128, bf16
 * q/K/V; page_size = 1 for the CSR page list (pkv_run) and a power of two up
 * to 1024 for block tables (pkv_block_table_run). Other shapes return
 * PKV_ERR_UNSUPPORTED.
 *
 * Layouts (all contiguous, row-major; bf16 as 16-bit patterns; device
 * pointers 16-byte aligned):
 *   q        bf16  [B, Hq, D]
 *   k_pool   bf16  [num_pages, page_size, Hkv, D]   (v_pool the same)
 *   kv_indptr int32 [B + 1]   (device copy: checked for non-NULL and length
 *            only, never read by the kernels, which take every sequence's
 *            token offset from the plan built from the host copy)
 *   kv_indices int32 [kv_indptr[B]], each in [0, num_pages)  (caller
 *            precondition, as in the page's kernel: not checked on device)
 *   out      bf16  [B, Hq, D]
 *   lse      fp32  [B, Hq], base 2
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,         /* null pointer, bad length, misaligned, non-finite scale */
  PKV_ERR_UNSUPPORTED = 2,         /* heads / dim / page size not compiled in */
  PKV_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below what the plan needs */
  PKV_ERR_PLAN_MISMATCH = 4,       /* call does not match the plan it names */
  PKV_ERR_HIP = 5                  /* a HIP runtime call or launch failed */
} pkv_status;

/* Opaque host object: the split-KV work partition of one batch. */
typedef struct pkv_plan pkv_plan;

/*
 * Bytes of device workspace a plan of this batch needs (work tables plus the
 * fp32 partials of split sequences). Same arguments as pkv_plan_create.
 * kv_indptr_host: host int32 [batch + 1], non-decreasing, kv_indptr_host[0] == 0.
 * num_cus: compute units to plan for; 0 queries the current HIP device.
 * allow_split: 0 gives one worker per sequence (nothing to merge).
 * chunk_tokens: tokens per worker; 0 uses one worker per CU (fewer for a
 * batch of under 128 tokens per worker).
 */
pkv_status pkv_workspace_size(const int32_t* kv_indptr_host, int32_t batch,
                              int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t page_size, int32_t num_cus, int32_t allow_split,
                              int32_t chunk_tokens, size_t* bytes);

/*
 * Build the split-KV partition of a batch (host work, O(batch)) and, when
 * `workspace` is non-NULL, enqueue the upload of its work tables into the
 * workspace on `stream` (a hipStream_t; NULL is the default stream). The
 * workspace must then be passed unchanged to pkv_run and pkv_merge; a NULL
 * workspace gives a host-only plan that can be exported but not run. The
 * plan records the batch shape; later calls that differ return
 * PKV_ERR_PLAN_MISMATCH (the plan-capture rule of the FlagGems
 * flash_mla_with_kvcache page, FlashMLASchedMeta). The caller keeps the device
 * kv_indptr equal to the host copy given here.
 * On success *plan receives a new object, freed with pkv_plan_destroy.
 */
pkv_status pkv_plan_create(const int32_t* kv_indptr_host, int32_t batch,
                           int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t page_size, int32_t num_cus, int32_t allow_split,
                           int32_t chunk_tokens, void* workspace, size_t workspace_bytes,
                           void* stream, pkv_plan** plan);

/* Frees a plan (NULL is ignored). Does not touch device memory. */
void pkv_plan_destroy(pkv_plan* plan);

/*
 * Bytes of device workspace this plan needs (the same number
 * pkv_workspace_size / pkv_block_table_workspace_size return for its batch),
 * so that a caller can make a host-only plan, size and allocate the
 * workspace, then bind it with pkv_plan_upload without building the
 * partition twice. PKV_ERR_INVALID_ARG for a NULL argument.
 */
pkv_status pkv_plan_workspace_size(const pkv_plan* plan, size_t* bytes);

/*
 * Enqueue the upload of the plan's work tables into `workspace` on `stream`
 * and bind the plan to it, exactly as passing the workspace to
 * pkv_plan_create would have (a plan may be re-bound to another workspace;
 * later runs must pass the workspace of the latest upload). The workspace must
 * hold pkv_plan_workspace_size bytes (PKV_ERR_WORKSPACE_TOO_SMALL otherwise)
 * and be 16-byte aligned (PKV_ERR_INVALID_ARG); PKV_ERR_HIP if the copy
 * cannot be enqueued. The host tables stay owned by the plan, so it must
 * outlive the copy (it does when it is destroyed after the stream's work).
 */
pkv_status pkv_plan_upload(pkv_plan* plan, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Which units run the decode kernel's two contractions (the scaled q.k scores
 * and the P.V product of the GQA page's decode steps) for later pkv_run /
 * pkv_block_table_run calls with this plan. PKV_ENGINE_MFMA (the default):
 * the matrix cores, with the 8 query heads of a KV head padded to 16 MFMA
 * columns. PKV_ENGINE_DOT2: the vector ALU, two bf16 products per lane and
 * instruction into fp32 (v_dot2c_f32_bf16). Both compute the same
 * definition with fp32 accumulation and P rounded to bf16; their results
 * differ only by rounding order. Any other value returns PKV_ERR_INVALID_ARG
 * and leaves the plan unchanged. Host only; the plan's tables do not change.
 */
enum { PKV_ENGINE_MFMA = 0, PKV_ENGINE_DOT2 = 1 };
pkv_status pkv_plan_set_engine(pkv_plan* plan, int32_t engine);

/*
 * Timing hook, for benchmarks and profilers that time the decode kernel with
 * events: while start_event and stop_event (hipEvent_t values the caller
 * created, with timing enabled) are set, the decode kernel enqueued by
 * pkv_run / pkv_block_table_run with this plan records its own start and end
 * time in them (hipExtLaunchKernel), so hipEventElapsedTime gives the
 * kernel's duration without the queue time of separately recorded events.
 * Both NULL (the default) launches without events; exactly one NULL returns
 * PKV_ERR_INVALID_ARG. The plan keeps the handles and does not own them: the
 * caller keeps the events alive while they are set. Not for launches under
 * stream capture. Host only.
 */
pkv_status pkv_plan_set_timing_events(pkv_plan* plan, void* start_event, void* stop_event);

/*
 * Copy the plan's integer tables to host memory:
 * [n_workers, n_segments, n_merges, n_slots], then n_workers + 1 offsets of
 * each worker's first segment, then n_segments records
 * (b, tok_begin, tok_end, slot) with token positions relative to sequence b
 * and slot -1 for a sequence written directly, then n_merges records
 * (b, first_slot, n_segments, 0) (n_segments 0 for an empty sequence).
 * Worker w (one workgroup) owns a contiguous run of the batch's tokens in
 * kv_indices order; the runs are balanced by cost (whole 32-token tiles plus
 * 32 tokens' worth for each segment), so a worker may hold fewer tokens when
 * it holds more segments. *needed receives the count of int32 values; dst may be
 * NULL to query it. Fails with PKV_ERR_INVALID_ARG when n_int32 is smaller
 * than that count.
 */
pkv_status pkv_plan_export(const pkv_plan* plan, int32_t* dst, size_t n_int32, size_t* needed);

/*
 * Enqueue the partial-decode kernel: one workgroup per worker of the plan.
 * Sequences inside one worker get their final out/lse; split sequences get
 * fp32 partials in the workspace, finished by pkv_merge. Shapes are passed so that they can be
 * checked against the plan: q is [q_batch, q_heads, q_dim], each pool is
 * [num_pages, page_size, pool_kv_heads, pool_dim], kv_indptr has indptr_len
 * entries and kv_indices has num_indices entries (must equal the plan's
 * kv_indptr[B]). sm_scale may be any finite value (the Python layer fills the
 * default 1/sqrt(head_dim)): the definition above holds for every real scale,
 * 0 giving equal weights (the mean of the V rows) and a negative scale
 * reversing the order of the scores; NaN or +-inf returns PKV_ERR_INVALID_ARG.
 */
pkv_status pkv_run(const pkv_plan* plan,
                   const void* q, int32_t q_batch, int32_t q_heads, int32_t q_dim,
                   const void* k_pool, const void* v_pool, int64_t num_pages,
                   int32_t page_size, int32_t pool_kv_heads, int32_t pool_dim,
                   const int32_t* kv_indptr, int64_t indptr_len,
                   const int32_t* kv_indices, int64_t num_indices,
                   float sm_scale, void* workspace, size_t workspace_bytes,
                   void* out, float* lse, void* stream);

/*
 * Paged decode with pages of several tokens found through a block table
 * (FlagGems flash_mla_with_kvcache page, _dense_decode_kernel: the page from
 * the table, the slot from the remainder, tokens past the sequence length
 * masked). Sequence b has seq_lens[b] tokens; its token j is slot
 * j % page_size of page block_table[b, j / page_size], so the last page may be
 * partly filled. The attention itself is the one stated at the top of this
 * file.
 *
 * pkv_block_table_workspace_size / pkv_block_table_plan_create take the host
 * int32 sequence lengths seq_lens_host [batch] (each >= 0, sum < 2^31) in
 * place of kv_indptr_host; every other argument means what it means for
 * pkv_workspace_size / pkv_plan_create. The plan fixes the lengths: the
 * device never reads them, so a plan is made per batch of lengths.
 *
 * pkv_block_table_run enqueues the partial decode for such a plan (pkv_run
 * rejects it with PKV_ERR_PLAN_MISMATCH, and this call rejects a CSR plan).
 * block_table: device int32 [table_rows, table_cols], row-major; table_rows
 * must equal the batch and table_cols must be at least the most pages any
 * sequence needs, ceil(seq_lens[b] / page_size). Only the first
 * ceil(seq_lens[b] / page_size) entries of row b are read, and each must be a
 * page in [0, num_pages) (caller precondition, not checked on device); other
 * entries may hold anything. The pool [num_pages, page_size, Hkv, D] may hold
 * at most 2^31 - 1 token rows. Finish with pkv_merge as after pkv_run.
 */
pkv_status pkv_block_table_workspace_size(const int32_t* seq_lens_host, int32_t batch,
                                          int32_t num_qo_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t page_size, int32_t num_cus,
                                          int32_t allow_split, int32_t chunk_tokens,
                                          size_t* bytes);
pkv_status pkv_block_table_plan_create(const int32_t* seq_lens_host, int32_t batch,
                                       int32_t num_qo_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t page_size, int32_t num_cus,
                                       int32_t allow_split, int32_t chunk_tokens, void* workspace,
                                       size_t workspace_bytes, void* stream, pkv_plan** plan);
pkv_status pkv_block_table_run(const pkv_plan* plan,
                               const void* q, int32_t q_batch, int32_t q_heads, int32_t q_dim,
                               const void* k_pool, const void* v_pool, int64_t num_pages,
                               int32_t page_size, int32_t pool_kv_heads, int32_t pool_dim,
                               const int32_t* block_table, int32_t table_rows,
                               int32_t table_cols, float sm_scale, void* workspace,
                               size_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * Enqueue the LSE merge of the sequences the plan split (and the zero output
 * of empty sequences); always call it after pkv_run, on the same stream with
 * the same workspace. Per (sequence, head): lse* = max_i lse_i,
 * w_i = 2^(lse_i - lse*), out = sum_i w_i o_i / sum_i w_i,
 * lse = lse* + log2(sum_i w_i); no pieces (or all -inf) gives out = 0,
 * lse = -inf. It enqueues nothing when there is nothing to merge.
 */
pkv_status pkv_merge(const pkv_plan* plan, void* workspace, size_t workspace_bytes,
                     void* out, float* lse, void* stream);

/*
 * KV append (vLLM fork qsa.py page, _store_qsa_rows_kernel and
 * qsa_store_cache_rows): store n_rows new K and V rows into the pools at
 * flat slot positions. Row i (k_rows / v_rows, bf16 [n_rows, num_kv_heads,
 * head_dim], contiguous) goes to page slot / page_size, position
 * slot % page_size of k_pool / v_pool (bf16 [num_pages, page_size,
 * num_kv_heads, head_dim]) with slot = slot_mapping[i] (device int64
 * [n_rows]); a slot outside [0, num_pages * page_size), e.g. -1 for padding,
 * stores nothing. The rows are copied bit for bit. Valid slots should be
 * distinct: rows that name the same slot race with nothing ordering their
 * stores, so each 16-byte unit of that slot ends up holding the same unit of
 * one of those rows (units of one slot, and its K and V, may come from
 * different rows). Any head count and head_dim whose row is a multiple of 16
 * bytes (at most 1 MiB) is accepted; n_rows <= 2^25. Pools and rows 16-byte
 * aligned, slot_mapping 8-byte aligned. Asynchronous on `stream`; n_rows = 0
 * enqueues nothing.
 */
pkv_status pkv_append_kv(void* k_pool, void* v_pool, int64_t num_pages, int32_t page_size,
                         int32_t num_kv_heads, int32_t head_dim, const void* k_rows,
                         const void* v_rows, const int64_t* slot_mapping, int64_t n_rows,
                         void* stream);

/*
 * Index-gather latent-attention decode (FlagGems flash_mla_with_kvcache page,
 * _sparse_decode_kernel in its bf16 mode). Row b attends to the pool rows
 * kv_pool[t] for every entry t = indices[b, i] with 0 <= t < pool_tokens;
 * other entries (e.g. -1) are masked and contribute nothing. Scores use all
 * d_qk dims; values are the first d_v dims of the same row:
 *     out[b,h] = sum_t exp(s_t) kv[t, :d_v] / sum_t exp(s_t),
 *     s_t = sm_scale * dot(q[b,h,:], kv[t,:]),   lse[b,h] = log2 sum_t exp(s_t)
 * and out = 0, lse = -inf when no entry is valid.
 * Optional (NULL = off), device pointers:
 *   topk_length int32 [batch]: row b reads only its first
 *     min(max(topk_length[b], 0), topk) entries (HAVE_TOPK_LENGTH on the page);
 *   attn_sink fp32 [num_qo_heads]: a logit in the natural-log units of
 *     sm_scale * q.k that joins the denominator with no value,
 *     out[b,h] = sum_t exp(s_t) kv[t, :d_v] / (sum_t exp(s_t) + exp(attn_sink[h]))
 *     (HAVE_ATTN_SINK); lse stays log2 sum_t exp(s_t), the entries alone, as
 *     the page stores it before applying the sink.
 * Layouts: q bf16 [batch, num_qo_heads, d_qk]; kv_pool bf16 [pool_tokens, d_qk];
 * indices int32 [batch, topk]; out bf16 [batch, num_qo_heads, d_v];
 * lse fp32 [batch, num_qo_heads]. Compiled for d_qk = 576, d_v = 512 and
 * num_qo_heads a multiple of 16 up to 128. workspace: device scratch of
 * pkv_gather_mla_workspace_size bytes. Degenerate shapes are valid: with
 * topk = 0 (indices may then be NULL) or pool_tokens = 0 (kv_pool may then
 * be NULL) every row has no valid entry and gets out 0, lse -inf; batch = 0
 * enqueues nothing.
 */
pkv_status pkv_gather_mla_workspace_size(int32_t batch, int32_t num_qo_heads, int32_t d_qk,
                                         int32_t d_v, int32_t topk, size_t* bytes);
pkv_status pkv_gather_mla(const void* q, const void* kv_pool, int64_t pool_tokens,
                          const int32_t* indices, int32_t topk, int32_t batch,
                          int32_t num_qo_heads, int32_t d_qk, int32_t d_v, float sm_scale,
                          const float* attn_sink, const int32_t* topk_length, void* workspace,
                          size_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * The bf16 gather above without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid allocation). Same arguments as pkv_gather_mla minus the workspace;
 * same results, bit for bit. The fp32 partials live in a device array the
 * library holds on each GPU it runs on (48 MiB, kept until the process ends),
 * found on the first call with that GPU current. A shape whose partials need
 * more than that (pkv_gather_mla_workspace_size bytes > 48 MiB) returns
 * PKV_ERR_UNSUPPORTED before any HIP call. The call allocates nothing. Every
 * call on one GPU shares its scratch: calls that overlap in time on one GPU
 * (different streams, or threads without ordering) race and may return wrong
 * results; calls ordered on one stream do not.
 */
pkv_status pkv_gather_mla_noalloc(const void* q, const void* kv_pool, int64_t pool_tokens,
                                  const int32_t* indices, int32_t topk, int32_t batch,
                                  int32_t num_qo_heads, int32_t d_qk, int32_t d_v, float sm_scale,
                                  const float* attn_sink, const int32_t* topk_length, void* out,
                                  float* lse, void* stream);

/*
 * The same gather over a pool of FP8 latent tokens (FlagGems
 * flash_mla_with_kvcache page, FP8 sparse mode): kv_pool is
 * [pool_tokens, 656] bytes per token: 512 OCP e4m3 ("e4m3fn") values, then 4
 * fp32 scales (scale k for values 128k .. 128k+127), then 64 bf16 values.
 * Each selected token is dequantised to 576 bf16 values, value i =
 * bf16_rne(fp32(e4m3[i]) * scale[i / 128]) for i < 512 and the stored bf16
 * values after; the attention is then the bf16 gather above (scores over all
 * 576 dims, values the first 512). Same arguments, options, workspace
 * (pkv_gather_mla_workspace_size) and errors; kv_pool 16-byte aligned.
 */
pkv_status pkv_gather_mla_fp8(const void* q, const void* kv_pool, int64_t pool_tokens,
                              const int32_t* indices, int32_t topk, int32_t batch,
                              int32_t num_qo_heads, int32_t d_qk, int32_t d_v, float sm_scale,
                              const float* attn_sink, const int32_t* topk_length,
                              void* workspace, size_t workspace_bytes, void* out, float* lse,
                              void* stream);

/* Static text for a status code. */
const char* pkv_status_string(pkv_status status);

/* Detail of the last failure on this thread ("" if none). */
const char* pkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
