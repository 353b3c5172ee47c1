// Split-KV work partition (host only). See plan.h for the rule.
#include "plan.h"

#include <algorithm>
#include <numeric>

namespace pkv {
namespace {

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t roundup(int64_t a, int64_t m) { return cdiv(a, m) * m; }

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
  p.total_tokens = kv_indptr[batch];
  int64_t chunk;
  if (!allow_split) {
    chunk = kNoSplitChunk;
  } else if (chunk_tokens > 0) {
    chunk = roundup(chunk_tokens, kTile);
  } else {
    const int64_t per_item =
        p.total_tokens > 0 ? cdiv(p.total_tokens, int64_t(num_cus) * kItemsPerCu) : 0;
    chunk = std::max<int64_t>(kMinChunk, roundup(per_item, kTile));
  }
  if (chunk > kNoSplitChunk) chunk = kNoSplitChunk;
  p.chunk = static_cast<int32_t>(chunk);

  std::vector<WorkItem> made;
  made.reserve(static_cast<size_t>(batch) + static_cast<size_t>(p.total_tokens / chunk) + 1);
  int32_t slot = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = int64_t(kv_indptr[b + 1]) - kv_indptr[b];
    if (n <= chunk) {
      made.push_back({b, 0, static_cast<int32_t>(n), -1});
      continue;
    }
    int64_t k = cdiv(n, chunk);
    const int64_t c = roundup(cdiv(n, k), kTile);
    k = cdiv(n, c);
    for (int64_t j = 0; j < k; ++j) {
      made.push_back({b, static_cast<int32_t>(j * c), static_cast<int32_t>(std::min((j + 1) * c, n)),
                      static_cast<int32_t>(slot + j)});
    }
    p.merges.push_back({b, slot, static_cast<int32_t>(k), 0});
    slot += static_cast<int32_t>(k);
  }
  p.n_slots = slot;
  // Longest items first so that the tail of the launch holds the short ones;
  // equal lengths keep their creation order.
  std::vector<size_t> order(made.size());
  std::iota(order.begin(), order.end(), size_t(0));
  std::stable_sort(order.begin(), order.end(), [&](size_t x, size_t y) {
    return (made[x].tok_end - made[x].tok_begin) > (made[y].tok_end - made[y].tok_begin);
  });
  p.items.reserve(made.size());
  for (size_t i : order) p.items.push_back(made[i]);
  *out = std::move(p);
  return true;
}

}  // namespace pkv
