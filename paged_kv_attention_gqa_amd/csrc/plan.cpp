// Split-KV work partition (host only). See plan.h for the rule.
#include "plan.h"

#include <algorithm>
#include <numeric>

namespace pkv {
namespace {

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

bool build_partition(const int32_t* kv_indptr, int32_t batch, int32_t num_cus,
                     bool allow_split, int32_t chunk_tokens, Partition* out, std::string* err) {
  if (batch < 0) { *err = "batch must be >= 0"; return false; }
  if (kv_indptr == nullptr) { *err = "kv_indptr is NULL"; return false; }
  if (kv_indptr[0] != 0) { *err = "kv_indptr[0] must be 0"; return false; }
  for (int32_t b = 0; b < batch; ++b) {
    if (kv_indptr[b + 1] < kv_indptr[b]) {
      *err = "kv_indptr must be non-decreasing (at b=" + std::to_string(b) + ")";
      return false;
    }
  }
  if (num_cus <= 0) { *err = "num_cus must be > 0"; return false; }
  if (chunk_tokens < 0) { *err = "chunk_tokens must be >= 0"; return false; }

  Partition p;
  const int64_t total = kv_indptr[batch];
  p.total_tokens = total;

  if (!allow_split) {
    // One worker per non-empty sequence, longest first; empty sequences are
    // merge records with no segments.
    std::vector<int32_t> order;
    for (int32_t b = 0; b < batch; ++b) {
      if (kv_indptr[b + 1] > kv_indptr[b]) order.push_back(b);
      else p.merges.push_back({b, 0, 0, 0});
    }
    std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
      return kv_indptr[x + 1] - kv_indptr[x] > kv_indptr[y + 1] - kv_indptr[y];
    });
    p.worker_ptr.push_back(0);
    for (int32_t b : order) {
      p.segments.push_back({b, 0, kv_indptr[b + 1] - kv_indptr[b], -1});
      p.worker_ptr.push_back(static_cast<int32_t>(p.segments.size()));
    }
    p.n_workers = static_cast<int32_t>(order.size());
    *out = std::move(p);
    return true;
  }

  int64_t workers;
  if (total == 0) {
    workers = 0;
  } else if (chunk_tokens > 0) {
    workers = cdiv(total, chunk_tokens);
  } else {
    workers = std::min<int64_t>(int64_t(num_cus) * kWorkersPerCu, cdiv(total, kMinWorkerTokens));
  }
  p.n_workers = static_cast<int32_t>(workers);
  // Worker w owns the tokens [start[w], start[w+1]), start[w] = w*total/workers,
  // each interior boundary moved (by at most 16 tokens) to the nearest
  // position that is a multiple of kTile tokens into its sequence, or to the
  // sequence's end, so that pieces of a sequence are whole tiles. Shares under
  // kSnapMinShare tokens are not moved.
  std::vector<int64_t> starts(static_cast<size_t>(workers) + 1);
  for (int64_t w = 0; w <= workers; ++w) starts[static_cast<size_t>(w)] = workers ? w * total / workers : 0;
  if (workers > 1 && total / workers >= kSnapMinShare) {
    for (int64_t w = 1; w < workers; ++w) {
      const int64_t pos = starts[static_cast<size_t>(w)];
      // sequence holding pos: last b with kv_indptr[b] <= pos
      const int32_t b = static_cast<int32_t>(
          std::upper_bound(kv_indptr, kv_indptr + batch + 1, static_cast<int32_t>(pos)) - kv_indptr - 1);
      const int64_t off = pos - kv_indptr[b];
      int64_t snapped = kv_indptr[b] + kTile * ((off + kTile / 2 - 1) / kTile);
      snapped = std::min<int64_t>(snapped, kv_indptr[b + 1]);
      starts[static_cast<size_t>(w)] = snapped;
    }
  }
  auto start = [&](int64_t w) { return starts[static_cast<size_t>(w)]; };

  std::vector<std::vector<Segment>> per_worker(static_cast<size_t>(workers));
  int32_t slot = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t lo = kv_indptr[b], hi = kv_indptr[b + 1];
    if (hi == lo) {
      p.merges.push_back({b, 0, 0, 0});
      continue;
    }
    // first worker whose range contains lo: largest w with start(w) <= lo
    int64_t w = std::min<int64_t>(workers - 1, (lo * workers) / total);
    while (w > 0 && start(w) > lo) --w;
    while (w + 1 < workers && start(w + 1) <= lo) ++w;
    const bool single = hi <= start(w + 1);
    int32_t k = 0;
    for (int64_t pos = lo; pos < hi; ++w) {
      const int64_t end = std::min<int64_t>(hi, start(w + 1));
      if (end > pos) {
        per_worker[static_cast<size_t>(w)].push_back(
            {b, static_cast<int32_t>(pos - lo), static_cast<int32_t>(end - lo),
             single ? -1 : slot + k});
        ++k;
      }
      pos = end;
    }
    if (!single) {
      p.merges.push_back({b, slot, k, 0});
      slot += k;
    }
  }
  p.n_slots = slot;
  p.worker_ptr.push_back(0);
  for (auto& segs : per_worker) {
    p.segments.insert(p.segments.end(), segs.begin(), segs.end());
    p.worker_ptr.push_back(static_cast<int32_t>(p.segments.size()));
  }
  *out = std::move(p);
  return true;
}

}  // namespace pkv
