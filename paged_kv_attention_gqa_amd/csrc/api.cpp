// C ABI of libpkv: argument checks, the plan object, workspace layout and
// kernel launches. Every check runs on the host before any HIP call, so a
// rejected call has no effect on the device.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "pkv.h"
#include "append.h"
#include "kernels.h"
#include "mla.h"
#include "plan.h"

struct pkv_plan {
  int32_t batch;
  int32_t num_qo_heads, num_kv_heads, head_dim, page_size;
  int32_t num_cus, allow_split;
  bool block_table;              // built from sequence lengths for pkv_block_table_run
  int64_t max_seq_pages;         // block-table plans: most pages any sequence needs
  pkv::Partition part;
  std::vector<int32_t> tables;   // worker offsets, segments, merge records, as uploaded
  pkv::FirstSegments firsts{};   // first segments' id positions, for the kernel arguments
  int32_t max_pieces = 0;        // most segments of one merge record
  pkv::DecodeEngine engine = pkv::DecodeEngine::kMfma;   // units of the decode contractions
  hipEvent_t start_event = nullptr, stop_event = nullptr;  // timing hook (both or neither)
  size_t off_wptr, off_segs, off_merges, off_part_o, off_part_lse, ws_bytes;
  void* workspace;               // device buffer the tables were uploaded to (or NULL)
};

namespace {

thread_local std::string g_last_error;

pkv_status fail(pkv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

pkv_status ok() {
  g_last_error.clear();
  return PKV_OK;
}

constexpr size_t kAlign = 256;
constexpr int64_t kMaxAppendRows = int64_t(1) << 25;   // 64 threads per row in a 32-bit grid
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int32_t kMaxPageSize = 1024;

// Page sizes: exactly 1 for the CSR list, a power of two up to kMaxPageSize
// for block tables.
pkv_status check_gqa_shape(int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t page_size, bool block_table) {
  if (num_qo_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || page_size <= 0)
    return fail(PKV_ERR_INVALID_ARG, "head counts, head_dim and page_size must be positive");
  if (num_qo_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_qo_heads (%d) must be a multiple of num_kv_heads (%d)",
                num_qo_heads, num_kv_heads);
  if (num_qo_heads != pkv::kHq)
    return fail(PKV_ERR_UNSUPPORTED, "expected num_qo_heads=%d, got %d", pkv::kHq, num_qo_heads);
  if (num_kv_heads != pkv::kHkv)
    return fail(PKV_ERR_UNSUPPORTED, "expected num_kv_heads=%d, got %d", pkv::kHkv, num_kv_heads);
  if (head_dim != pkv::kHeadDim)
    return fail(PKV_ERR_UNSUPPORTED, "expected head_dim=%d, got %d", pkv::kHeadDim, head_dim);
  if (!block_table && page_size != 1)
    return fail(PKV_ERR_UNSUPPORTED,
                "expected page_size=1 for a CSR page list, got %d (use the block-table calls)",
                page_size);
  if (block_table && (page_size > kMaxPageSize || (page_size & (page_size - 1)) != 0))
    return fail(PKV_ERR_UNSUPPORTED, "page_size must be a power of two <= %d, got %d",
                kMaxPageSize, page_size);
  return PKV_OK;
}

int32_t log2_exact(int32_t x) {
  int32_t s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

// CU count of the current device, queried once per device.
constexpr int kMaxDevices = 64;
std::atomic<int32_t> g_device_cus[kMaxDevices];

pkv_status resolve_cus(int32_t* num_cus) {
  if (*num_cus > 0) return PKV_OK;
  if (*num_cus < 0) return fail(PKV_ERR_INVALID_ARG, "num_cus must be >= 0");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < kMaxDevices) {
    const int32_t known = g_device_cus[dev].load(std::memory_order_relaxed);
    if (known > 0) {
      *num_cus = known;
      return PKV_OK;
    }
  }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < kMaxDevices) g_device_cus[dev].store(cus, std::memory_order_relaxed);
  *num_cus = cus;
  return PKV_OK;
}

// Builds the partition and the workspace layout of a plan (no device work).
// kv_indptr_host holds the token offsets of the sequences (for a block-table
// plan, the prefix sums of the sequence lengths).
pkv_status make_plan(const int32_t* kv_indptr_host, int32_t batch, int32_t num_qo_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t num_cus,
                     int32_t allow_split, int32_t chunk_tokens, bool block_table, pkv_plan* p) {
  if (kv_indptr_host == nullptr) return fail(PKV_ERR_INVALID_ARG, "kv_indptr_host is NULL");
  if (batch < 0) return fail(PKV_ERR_INVALID_ARG, "batch must be >= 0");
  pkv_status s = check_gqa_shape(num_qo_heads, num_kv_heads, head_dim, page_size, block_table);
  if (s != PKV_OK) return s;
  if (chunk_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "chunk_tokens must be >= 0");
  s = resolve_cus(&num_cus);
  if (s != PKV_OK) return s;
  std::string err;
  if (!pkv::build_partition(kv_indptr_host, batch, num_cus, allow_split != 0, chunk_tokens,
                            &p->part, &err))
    return fail(PKV_ERR_INVALID_ARG, "%s", err.c_str());
  p->batch = batch;
  p->num_qo_heads = num_qo_heads;
  p->num_kv_heads = num_kv_heads;
  p->head_dim = head_dim;
  p->page_size = page_size;
  p->num_cus = num_cus;
  p->allow_split = allow_split != 0;
  p->block_table = block_table;
  p->max_seq_pages = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = static_cast<int64_t>(kv_indptr_host[b + 1]) - kv_indptr_host[b];
    p->max_seq_pages = std::max<int64_t>(p->max_seq_pages, (n + page_size - 1) / page_size);
  }
  // Uploaded tables (all records 8 int32 = 32 bytes):
  // * worker w: (first segment's b, tok_begin, tok_end, slot, token offset of
  //   its sequence, s_begin, s_end, 0), so a workgroup starts its first
  //   segment after one load;
  // * segment s: (b, tok_begin, tok_end, slot, token offset of sequence b,
  //   0, 0, 0), so page ids are found without reading kv_indptr;
  // * merge records (b, first_slot, n_segments, 0).
  const pkv::Partition& pt = p->part;
  const size_t n_workers = static_cast<size_t>(pt.n_workers);
  const size_t n_segs = pt.segments.size();
  p->tables.resize(8 * (n_workers + n_segs) + 4 * pt.merges.size());
  int32_t* t = p->tables.data();
  for (size_t w = 0; w < n_workers; ++w, t += 8) {
    const int32_t sb = pt.worker_ptr[w];
    const int32_t se = pt.worker_ptr[w + 1];
    const pkv::Segment sg = sb < se ? pt.segments[static_cast<size_t>(sb)] : pkv::Segment{0, 0, 0, -1};
    t[0] = sg.b; t[1] = sg.tok_begin; t[2] = sg.tok_end; t[3] = sg.slot;
    t[4] = sb < se ? kv_indptr_host[sg.b] : 0; t[5] = sb; t[6] = se; t[7] = 0;
  }
  const size_t n_wrec = 8 * n_workers;
  // The first segment of the first kFirstArgWorkers workers, for the kernel
  // arguments (see kernels.h).
  const int32_t n_firsts = static_cast<int32_t>(std::min<size_t>(n_workers, pkv::kFirstArgWorkers));
  for (int32_t w = 0; w < n_firsts; ++w) {
    const int32_t* r = p->tables.data() + 8 * static_cast<size_t>(w);
    const bool has = r[5] < r[6];
    p->firsts.v[3 * w] = has ? (block_table ? r[0] : r[4] + r[1]) : 0;
    p->firsts.v[3 * w + 1] = has && block_table ? r[1] : 0;
    p->firsts.v[3 * w + 2] = has ? r[2] - r[1] : 0;
  }
  for (const auto& sg : pt.segments) {
    t[0] = sg.b; t[1] = sg.tok_begin; t[2] = sg.tok_end; t[3] = sg.slot;
    t[4] = kv_indptr_host[sg.b]; t[5] = 0; t[6] = 0; t[7] = 0;
    t += 8;
  }
  p->max_pieces = 0;
  for (const auto& m : pt.merges) {
    p->max_pieces = std::max(p->max_pieces, m.n_segments);
    t[0] = m.b; t[1] = m.first_slot; t[2] = m.n_segments; t[3] = m.pad;
    t += 4;
  }
  const size_t slots = static_cast<size_t>(p->part.n_slots);
  p->off_wptr = 0;
  p->off_segs = 4 * n_wrec;
  p->off_merges = p->off_segs + 32 * p->part.segments.size();
  p->off_part_o = align_up(p->off_merges + 16 * p->part.merges.size());
  p->off_part_lse = align_up(p->off_part_o + slots * num_qo_heads * head_dim * sizeof(float));
  p->ws_bytes = align_up(p->off_part_lse + slots * num_qo_heads * sizeof(float));
  p->workspace = nullptr;
  return PKV_OK;
}

// Token offsets (prefix sums) of block-table sequence lengths.
pkv_status offsets_from_lengths(const int32_t* seq_lens_host, int32_t batch,
                                std::vector<int32_t>* indptr) {
  if (seq_lens_host == nullptr && batch > 0)
    return fail(PKV_ERR_INVALID_ARG, "seq_lens_host is NULL");
  if (batch < 0) return fail(PKV_ERR_INVALID_ARG, "batch must be >= 0");
  indptr->assign(static_cast<size_t>(batch) + 1, 0);
  int64_t total = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (seq_lens_host[b] < 0)
      return fail(PKV_ERR_INVALID_ARG, "seq_lens[%d] = %d is negative", b, seq_lens_host[b]);
    total += seq_lens_host[b];
    if (total > INT32_MAX)
      return fail(PKV_ERR_INVALID_ARG, "the batch holds more than 2^31 - 1 tokens");
    (*indptr)[static_cast<size_t>(b) + 1] = static_cast<int32_t>(total);
  }
  return PKV_OK;
}

// Checks the workspace and enqueues the copy of the plan's tables into it;
// the plan is then bound to that workspace.
pkv_status upload_plan(pkv_plan* p, void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace == nullptr) return fail(PKV_ERR_INVALID_ARG, "workspace is NULL");
  if (workspace_bytes < p->ws_bytes)
    return fail(PKV_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, plan needs %zu",
                workspace_bytes, p->ws_bytes);
  if (!aligned16(workspace)) return fail(PKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (!p->tables.empty()) {
    hipError_t e = hipMemcpyAsync(workspace, p->tables.data(), p->tables.size() * sizeof(int32_t),
                                  hipMemcpyHostToDevice, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
      return fail(PKV_ERR_HIP, "uploading the plan tables: %s", hipGetErrorString(e));
  }
  p->workspace = workspace;
  return PKV_OK;
}

// Shared by pkv_plan_create and pkv_block_table_plan_create.
pkv_status create_plan(const int32_t* kv_indptr_host, int32_t batch, int32_t num_qo_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                       int32_t num_cus, int32_t allow_split, int32_t chunk_tokens,
                       bool block_table, void* workspace, size_t workspace_bytes, void* stream,
                       pkv_plan** plan) {
  if (plan == nullptr) return fail(PKV_ERR_INVALID_ARG, "plan is NULL");
  *plan = nullptr;
  pkv_plan* p = new (std::nothrow) pkv_plan();
  if (p == nullptr) return fail(PKV_ERR_INVALID_ARG, "out of host memory");
  pkv_status s = make_plan(kv_indptr_host, batch, num_qo_heads, num_kv_heads, head_dim,
                           page_size, num_cus, allow_split, chunk_tokens, block_table, p);
  if (s != PKV_OK) {
    delete p;
    return s;
  }
  if (workspace != nullptr) {
    s = upload_plan(p, workspace, workspace_bytes, stream);
    if (s != PKV_OK) {
      delete p;
      return s;
    }
  }
  *plan = p;
  return ok();
}

// Checks shared by pkv_run and pkv_block_table_run: the call against the
// plan, pointers and alignment.
pkv_status check_run(const pkv_plan* plan, bool block_table, const void* q, int32_t q_batch,
                     int32_t q_heads, int32_t q_dim, const void* k_pool, const void* v_pool,
                     int64_t num_pages, int32_t page_size, int32_t pool_kv_heads,
                     int32_t pool_dim, float sm_scale, const void* out, const float* lse) {
  if (plan == nullptr) return fail(PKV_ERR_INVALID_ARG, "plan is NULL");
  if (plan->block_table != block_table)
    return fail(PKV_ERR_PLAN_MISMATCH, block_table
                    ? "plan was made for a CSR page list (pkv_plan_create); use pkv_run"
                    : "plan was made for a block table (pkv_block_table_plan_create); "
                      "use pkv_block_table_run");
  pkv_status s = check_gqa_shape(q_heads, pool_kv_heads, q_dim, page_size, block_table);
  if (s != PKV_OK) return s;
  if (pool_dim != q_dim)
    return fail(PKV_ERR_INVALID_ARG, "pool head_dim %d differs from q head_dim %d", pool_dim, q_dim);
  if (q_batch != plan->batch || q_heads != plan->num_qo_heads || pool_kv_heads != plan->num_kv_heads ||
      q_dim != plan->head_dim || page_size != plan->page_size)
    return fail(PKV_ERR_PLAN_MISMATCH,
                "call shape (B=%d, Hq=%d, Hkv=%d, D=%d, ps=%d) differs from the plan's "
                "(B=%d, Hq=%d, Hkv=%d, D=%d, ps=%d)",
                q_batch, q_heads, pool_kv_heads, q_dim, page_size, plan->batch,
                plan->num_qo_heads, plan->num_kv_heads, plan->head_dim, plan->page_size);
  if (num_pages < 0) return fail(PKV_ERR_INVALID_ARG, "num_pages must be >= 0");
  if (plan->part.total_tokens > 0 && num_pages == 0)
    return fail(PKV_ERR_INVALID_ARG, "the batch has tokens but the pool has no pages");
  if (num_pages * static_cast<int64_t>(page_size) > INT32_MAX)
    return fail(PKV_ERR_UNSUPPORTED, "the pool holds more than 2^31 - 1 token rows");
  if (!std::isfinite(sm_scale)) return fail(PKV_ERR_INVALID_ARG, "sm_scale must be finite");
  if (plan->batch > 0) {
    if (q == nullptr || out == nullptr || lse == nullptr)
      return fail(PKV_ERR_INVALID_ARG, "q, out and lse must be non-NULL");
    if (plan->part.total_tokens > 0 && (k_pool == nullptr || v_pool == nullptr))
      return fail(PKV_ERR_INVALID_ARG, "k_pool and v_pool must be non-NULL");
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
      return fail(PKV_ERR_INVALID_ARG, "q, k_pool, v_pool and out must be 16-byte aligned");
  }
  return PKV_OK;
}

// Checks the workspace against the plan, then enqueues the decode kernel.
pkv_status launch_run(const pkv_plan* plan, const void* q, const void* k_pool, const void* v_pool,
                      const pkv::KvAddressing& addr, float sm_scale, void* workspace,
                      size_t workspace_bytes, void* out, float* lse, void* stream) {
  if (plan->workspace == nullptr)
    return fail(PKV_ERR_PLAN_MISMATCH, "host-only plan (created without a workspace)");
  if (workspace != plan->workspace)
    return fail(PKV_ERR_PLAN_MISMATCH, "workspace differs from the one the plan was uploaded to");
  if (workspace_bytes < plan->ws_bytes)
    return fail(PKV_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, plan needs %zu",
                workspace_bytes, plan->ws_bytes);
  if (plan->part.n_workers == 0) return ok();
  char* ws = static_cast<char*>(workspace);
  const float log2e = 1.4426950408889634f;
  hipError_t e = pkv::launch_decode_partial(
      reinterpret_cast<const int32_t*>(ws + plan->off_wptr),
      reinterpret_cast<const int32_t*>(ws + plan->off_segs), plan->firsts,
      plan->part.n_workers,
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_pool),
      static_cast<const uint16_t*>(v_pool), addr, sm_scale * log2e, static_cast<uint16_t*>(out),
      lse, reinterpret_cast<float*>(ws + plan->off_part_o),
      reinterpret_cast<float*>(ws + plan->off_part_lse), plan->engine, plan->start_event,
      plan->stop_event, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

namespace {

pkv_status gather_common(const void* q, const void* kv_pool, bool fp8_pool, int64_t pool_tokens,
                         const int32_t* indices, int32_t topk, int32_t batch, int32_t num_qo_heads,
                         int32_t d_qk, int32_t d_v, float sm_scale, const float* attn_sink,
                         const int32_t* topk_length, void* workspace, size_t workspace_bytes,
                         void* out, float* lse, void* stream) {
  std::string err;
  size_t need = 0;
  int code = pkv::mla_workspace_bytes(batch, num_qo_heads, d_qk, d_v, topk, &need, &err);
  if (code != 0) return fail(static_cast<pkv_status>(code), "%s", err.c_str());
  if (pool_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "pool_tokens must be >= 0");
  if (!std::isfinite(sm_scale)) return fail(PKV_ERR_INVALID_ARG, "sm_scale must be finite");
  if (batch == 0) return ok();
  if (q == nullptr || out == nullptr || lse == nullptr)
    return fail(PKV_ERR_INVALID_ARG, "q, out and lse must be non-NULL");
  if (topk > 0 && indices == nullptr) return fail(PKV_ERR_INVALID_ARG, "indices is NULL");
  if (pool_tokens > 0 && kv_pool == nullptr) return fail(PKV_ERR_INVALID_ARG, "kv_pool is NULL");
  if (!aligned16(q) || !aligned16(kv_pool) || !aligned16(out) || !aligned16(workspace))
    return fail(PKV_ERR_INVALID_ARG, "q, kv_pool, out and workspace must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(attn_sink) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(topk_length) & 3u) != 0)
    return fail(PKV_ERR_INVALID_ARG, "attn_sink and topk_length must be 4-byte aligned");
  if (need > 0 && workspace == nullptr) return fail(PKV_ERR_INVALID_ARG, "workspace is NULL");
  if (workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, gather needs %zu",
                workspace_bytes, need);
  hipError_t e = pkv::launch_gather_mla(
      static_cast<const uint16_t*>(q), kv_pool, fp8_pool, pool_tokens, indices, topk, batch,
      num_qo_heads, sm_scale, attn_sink, topk_length, workspace, static_cast<uint16_t*>(out), lse,
      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "gather launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* pkv_status_string(pkv_status status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape";
    case PKV_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PKV_ERR_PLAN_MISMATCH: return "call does not match the plan";
    case PKV_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* pkv_last_error(void) { return g_last_error.c_str(); }

pkv_status pkv_workspace_size(const int32_t* kv_indptr_host, int32_t batch, int32_t num_qo_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                              int32_t num_cus, int32_t allow_split, int32_t chunk_tokens,
                              size_t* bytes) {
  if (bytes == nullptr) return fail(PKV_ERR_INVALID_ARG, "bytes is NULL");
  pkv_plan p;
  pkv_status s = make_plan(kv_indptr_host, batch, num_qo_heads, num_kv_heads, head_dim,
                           page_size, num_cus, allow_split, chunk_tokens, false, &p);
  if (s != PKV_OK) return s;
  *bytes = p.ws_bytes;
  return ok();
}

pkv_status pkv_plan_create(const int32_t* kv_indptr_host, int32_t batch, int32_t num_qo_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                           int32_t num_cus, int32_t allow_split, int32_t chunk_tokens,
                           void* workspace, size_t workspace_bytes, void* stream,
                           pkv_plan** plan) {
  return create_plan(kv_indptr_host, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                     num_cus, allow_split, chunk_tokens, false, workspace, workspace_bytes, stream,
                     plan);
}

pkv_status pkv_block_table_workspace_size(const int32_t* seq_lens_host, int32_t batch,
                                          int32_t num_qo_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t page_size, int32_t num_cus,
                                          int32_t allow_split, int32_t chunk_tokens,
                                          size_t* bytes) {
  if (bytes == nullptr) return fail(PKV_ERR_INVALID_ARG, "bytes is NULL");
  std::vector<int32_t> indptr;
  pkv_status s = offsets_from_lengths(seq_lens_host, batch, &indptr);
  if (s != PKV_OK) return s;
  pkv_plan p;
  s = make_plan(indptr.data(), batch, num_qo_heads, num_kv_heads, head_dim, page_size, num_cus,
                allow_split, chunk_tokens, true, &p);
  if (s != PKV_OK) return s;
  *bytes = p.ws_bytes;
  return ok();
}

pkv_status pkv_block_table_plan_create(const int32_t* seq_lens_host, int32_t batch,
                                       int32_t num_qo_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t page_size, int32_t num_cus,
                                       int32_t allow_split, int32_t chunk_tokens, void* workspace,
                                       size_t workspace_bytes, void* stream, pkv_plan** plan) {
  if (plan == nullptr) return fail(PKV_ERR_INVALID_ARG, "plan is NULL");
  *plan = nullptr;
  std::vector<int32_t> indptr;
  pkv_status s = offsets_from_lengths(seq_lens_host, batch, &indptr);
  if (s != PKV_OK) return s;
  return create_plan(indptr.data(), batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                     num_cus, allow_split, chunk_tokens, true, workspace, workspace_bytes, stream,
                     plan);
}

void pkv_plan_destroy(pkv_plan* plan) { delete plan; }

pkv_status pkv_plan_workspace_size(const pkv_plan* plan, size_t* bytes) {
  if (plan == nullptr || bytes == nullptr) return fail(PKV_ERR_INVALID_ARG, "plan and bytes must be non-NULL");
  *bytes = plan->ws_bytes;
  return ok();
}

pkv_status pkv_plan_upload(pkv_plan* plan, void* workspace, size_t workspace_bytes, void* stream) {
  if (plan == nullptr) return fail(PKV_ERR_INVALID_ARG, "plan is NULL");
  const pkv_status s = upload_plan(plan, workspace, workspace_bytes, stream);
  return s == PKV_OK ? ok() : s;
}

pkv_status pkv_plan_set_engine(pkv_plan* plan, int32_t engine) {
  if (plan == nullptr) return fail(PKV_ERR_INVALID_ARG, "plan is NULL");
  if (engine != PKV_ENGINE_MFMA && engine != PKV_ENGINE_DOT2)
    return fail(PKV_ERR_INVALID_ARG, "engine must be PKV_ENGINE_MFMA (0) or PKV_ENGINE_DOT2 (1), got %d",
                engine);
  plan->engine = static_cast<pkv::DecodeEngine>(engine);
  return ok();
}

pkv_status pkv_plan_set_timing_events(pkv_plan* plan, void* start_event, void* stop_event) {
  if (plan == nullptr) return fail(PKV_ERR_INVALID_ARG, "plan is NULL");
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(PKV_ERR_INVALID_ARG, "start_event and stop_event must both be set or both NULL");
  plan->start_event = static_cast<hipEvent_t>(start_event);
  plan->stop_event = static_cast<hipEvent_t>(stop_event);
  return ok();
}

pkv_status pkv_plan_export(const pkv_plan* plan, int32_t* dst, size_t n_int32, size_t* needed) {
  if (plan == nullptr) return fail(PKV_ERR_INVALID_ARG, "plan is NULL");
  const auto& pt = plan->part;
  const size_t count = 4 + pt.worker_ptr.size() + 4 * (pt.segments.size() + pt.merges.size());
  if (needed != nullptr) *needed = count;
  if (dst == nullptr) return ok();
  if (n_int32 < count)
    return fail(PKV_ERR_INVALID_ARG, "export needs %zu int32 values, got %zu", count, n_int32);
  int32_t* d = dst;
  *d++ = pt.n_workers;
  *d++ = static_cast<int32_t>(pt.segments.size());
  *d++ = static_cast<int32_t>(pt.merges.size());
  *d++ = pt.n_slots;
  for (int32_t v : pt.worker_ptr) *d++ = v;
  for (const auto& sg : pt.segments) {
    *d++ = sg.b; *d++ = sg.tok_begin; *d++ = sg.tok_end; *d++ = sg.slot;
  }
  for (const auto& m : pt.merges) {
    *d++ = m.b; *d++ = m.first_slot; *d++ = m.n_segments; *d++ = m.pad;
  }
  return ok();
}

pkv_status pkv_run(const pkv_plan* plan, const void* q, int32_t q_batch, int32_t q_heads,
                   int32_t q_dim, const void* k_pool, const void* v_pool, int64_t num_pages,
                   int32_t page_size, int32_t pool_kv_heads, int32_t pool_dim,
                   const int32_t* kv_indptr, int64_t indptr_len, const int32_t* kv_indices,
                   int64_t num_indices, float sm_scale, void* workspace, size_t workspace_bytes,
                   void* out, float* lse, void* stream) {
  pkv_status s = check_run(plan, false, q, q_batch, q_heads, q_dim, k_pool, v_pool, num_pages,
                           page_size, pool_kv_heads, pool_dim, sm_scale, out, lse);
  if (s != PKV_OK) return s;
  if (indptr_len != static_cast<int64_t>(plan->batch) + 1)
    return fail(PKV_ERR_INVALID_ARG, "kv_indptr has %lld entries, expected batch + 1 = %d",
                static_cast<long long>(indptr_len), plan->batch + 1);
  if (num_indices != plan->part.total_tokens)
    return fail(PKV_ERR_INVALID_ARG, "kv_indices has %lld entries but kv_indptr[B] = %lld",
                static_cast<long long>(num_indices), static_cast<long long>(plan->part.total_tokens));
  if (plan->batch > 0 && kv_indptr == nullptr)
    return fail(PKV_ERR_INVALID_ARG, "kv_indptr must be non-NULL");
  if (num_indices > 0 && kv_indices == nullptr)
    return fail(PKV_ERR_INVALID_ARG, "kv_indices must be non-NULL");
  const pkv::KvAddressing addr{kv_indptr, kv_indices, 0, 0};
  return launch_run(plan, q, k_pool, v_pool, addr, sm_scale, workspace, workspace_bytes, out, lse,
                    stream);
}

pkv_status pkv_block_table_run(const pkv_plan* plan, const void* q, int32_t q_batch,
                               int32_t q_heads, int32_t q_dim, const void* k_pool,
                               const void* v_pool, int64_t num_pages, int32_t page_size,
                               int32_t pool_kv_heads, int32_t pool_dim,
                               const int32_t* block_table, int32_t table_rows,
                               int32_t table_cols, float sm_scale, void* workspace,
                               size_t workspace_bytes, void* out, float* lse, void* stream) {
  pkv_status s = check_run(plan, true, q, q_batch, q_heads, q_dim, k_pool, v_pool, num_pages,
                           page_size, pool_kv_heads, pool_dim, sm_scale, out, lse);
  if (s != PKV_OK) return s;
  if (table_rows != plan->batch)
    return fail(PKV_ERR_INVALID_ARG, "block_table has %d rows, expected batch = %d", table_rows,
                plan->batch);
  if (table_cols < 0 || table_cols < plan->max_seq_pages)
    return fail(PKV_ERR_INVALID_ARG,
                "block_table has %d columns but the longest sequence needs %lld pages",
                table_cols, static_cast<long long>(plan->max_seq_pages));
  if (plan->part.total_tokens > 0 && block_table == nullptr)
    return fail(PKV_ERR_INVALID_ARG, "block_table must be non-NULL");
  const pkv::KvAddressing addr{nullptr, block_table, table_cols, log2_exact(page_size)};
  return launch_run(plan, q, k_pool, v_pool, addr, sm_scale, workspace, workspace_bytes, out, lse,
                    stream);
}

pkv_status pkv_merge(const pkv_plan* plan, void* workspace, size_t workspace_bytes, void* out,
                     float* lse, void* stream) {
  if (plan == nullptr) return fail(PKV_ERR_INVALID_ARG, "plan is NULL");
  if (plan->part.merges.empty()) return ok();
  if (out == nullptr || lse == nullptr) return fail(PKV_ERR_INVALID_ARG, "out and lse must be non-NULL");
  if (!aligned16(out)) return fail(PKV_ERR_INVALID_ARG, "out must be 16-byte aligned");
  if (plan->workspace == nullptr || workspace != plan->workspace)
    return fail(PKV_ERR_PLAN_MISMATCH, "workspace differs from the one the plan was uploaded to");
  if (workspace_bytes < plan->ws_bytes)
    return fail(PKV_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, plan needs %zu",
                workspace_bytes, plan->ws_bytes);
  char* ws = static_cast<char*>(workspace);
  hipError_t e = pkv::launch_merge(reinterpret_cast<const int32_t*>(ws + plan->off_merges),
                                   plan->tables.data() + plan->off_merges / sizeof(int32_t),
                                   static_cast<int32_t>(plan->part.merges.size()),
                                   plan->max_pieces,
                                   reinterpret_cast<const float*>(ws + plan->off_part_o),
                                   reinterpret_cast<const float*>(ws + plan->off_part_lse),
                                   static_cast<uint16_t*>(out), lse, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "merge launch: %s", hipGetErrorString(e));
  return ok();
}

pkv_status pkv_append_kv(void* k_pool, void* v_pool, int64_t num_pages, int32_t page_size,
                         int32_t num_kv_heads, int32_t head_dim, const void* k_rows,
                         const void* v_rows, const int64_t* slot_mapping, int64_t n_rows,
                         void* stream) {
  if (num_pages < 0 || page_size <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PKV_ERR_INVALID_ARG,
                "num_pages must be >= 0 and page_size, num_kv_heads, head_dim positive");
  const int64_t row_bytes = static_cast<int64_t>(num_kv_heads) * head_dim * 2;
  if (row_bytes % 16 != 0 || row_bytes > (1 << 20))
    return fail(PKV_ERR_UNSUPPORTED,
                "a K/V row (num_kv_heads * head_dim bf16) must be a multiple of 16 bytes and at "
                "most 1 MiB, got %lld bytes", static_cast<long long>(row_bytes));
  if (num_pages > INT64_MAX / page_size / row_bytes)
    return fail(PKV_ERR_INVALID_ARG, "pool size overflows");
  if (n_rows < 0 || n_rows > kMaxAppendRows)
    return fail(PKV_ERR_INVALID_ARG, "n_rows must be in [0, %lld], got %lld",
                static_cast<long long>(kMaxAppendRows), static_cast<long long>(n_rows));
  if (n_rows == 0) return ok();
  if (k_rows == nullptr || v_rows == nullptr || slot_mapping == nullptr)
    return fail(PKV_ERR_INVALID_ARG, "k_rows, v_rows and slot_mapping must be non-NULL");
  if (num_pages > 0 && (k_pool == nullptr || v_pool == nullptr))
    return fail(PKV_ERR_INVALID_ARG, "k_pool and v_pool must be non-NULL");
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_rows) || !aligned16(v_rows) ||
      (reinterpret_cast<uintptr_t>(slot_mapping) & 7u) != 0)
    return fail(PKV_ERR_INVALID_ARG,
                "pools and rows must be 16-byte aligned and slot_mapping 8-byte aligned");
  hipError_t e = pkv::launch_append(k_pool, v_pool, num_pages * page_size, k_rows, v_rows,
                                    slot_mapping, n_rows, static_cast<int32_t>(row_bytes),
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "append launch: %s", hipGetErrorString(e));
  return ok();
}

pkv_status pkv_gather_mla_workspace_size(int32_t batch, int32_t num_qo_heads, int32_t d_qk,
                                         int32_t d_v, int32_t topk, size_t* bytes) {
  if (bytes == nullptr) return fail(PKV_ERR_INVALID_ARG, "bytes is NULL");
  std::string err;
  size_t need = 0;
  const int code = pkv::mla_workspace_bytes(batch, num_qo_heads, d_qk, d_v, topk, &need, &err);
  if (code != 0) return fail(static_cast<pkv_status>(code), "%s", err.c_str());
  *bytes = need;
  return ok();
}

pkv_status pkv_gather_mla(const void* q, const void* kv_pool, int64_t pool_tokens,
                          const int32_t* indices, int32_t topk, int32_t batch,
                          int32_t num_qo_heads, int32_t d_qk, int32_t d_v, float sm_scale,
                          const float* attn_sink, const int32_t* topk_length, void* workspace,
                          size_t workspace_bytes, void* out, float* lse, void* stream) {
  return gather_common(q, kv_pool, false, pool_tokens, indices, topk, batch, num_qo_heads, d_qk,
                       d_v, sm_scale, attn_sink, topk_length, workspace, workspace_bytes, out,
                       lse, stream);
}

pkv_status pkv_gather_mla_noalloc(const void* q, const void* kv_pool, int64_t pool_tokens,
                                  const int32_t* indices, int32_t topk, int32_t batch,
                                  int32_t num_qo_heads, int32_t d_qk, int32_t d_v, float sm_scale,
                                  const float* attn_sink, const int32_t* topk_length, void* out,
                                  float* lse, void* stream) {
  std::string err;
  size_t need = 0;
  const int code = pkv::mla_workspace_bytes(batch, num_qo_heads, d_qk, d_v, topk, &need, &err);
  if (code != 0) return fail(static_cast<pkv_status>(code), "%s", err.c_str());
  if (need > pkv::kMlaScratchBytes)
    return fail(PKV_ERR_UNSUPPORTED,
                "this gather needs %zu bytes of partials; the library's device scratch holds %zu "
                "(use pkv_gather_mla with a workspace)",
                need, pkv::kMlaScratchBytes);
  void* scratch = nullptr;
  if (need > 0 && batch > 0) {
    const hipError_t e = pkv::mla_scratch(&scratch);
    if (e != hipSuccess)
      return fail(PKV_ERR_HIP, "locating the device scratch: %s", hipGetErrorString(e));
  }
  return gather_common(q, kv_pool, false, pool_tokens, indices, topk, batch, num_qo_heads, d_qk,
                       d_v, sm_scale, attn_sink, topk_length, scratch, need, out, lse, stream);
}

pkv_status pkv_gather_mla_fp8(const void* q, const void* kv_pool, int64_t pool_tokens,
                              const int32_t* indices, int32_t topk, int32_t batch,
                              int32_t num_qo_heads, int32_t d_qk, int32_t d_v, float sm_scale,
                              const float* attn_sink, const int32_t* topk_length,
                              void* workspace, size_t workspace_bytes, void* out, float* lse,
                              void* stream) {
  return gather_common(q, kv_pool, true, pool_tokens, indices, topk, batch, num_qo_heads, d_qk,
                       d_v, sm_scale, attn_sink, topk_length, workspace, workspace_bytes, out,
                       lse, stream);
}

}  // extern "C"
