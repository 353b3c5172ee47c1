// Split-KV work partition (host only). See plan.h for the rule.
#include "plan.h"

#include <algorithm>
#include <climits>
#include <numeric>

namespace pkv {
namespace {

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Cost of decoding n tokens of one sequence as one segment, in tokens: its
// tiles plus the fixed price of starting a segment.
int64_t piece_cost(int64_t n) { return cdiv(n, kTile) * kTile + kSegmentCost; }

struct Piece {
  int64_t w;
  int32_t b, lo, hi;
};

// Fills workers of cost `budget` with the sequences in order: the rest of a
// sequence goes whole to the current worker if it fits, else the worker takes
// the whole tiles that fit and the next worker continues. Returns the number
// of workers used (-1 if the budget cannot hold one tile and a segment) and,
// if `pieces` is given, the pieces in order.
int64_t greedy_fill(const int32_t* kv_indptr, int32_t batch, int64_t budget,
                    std::vector<Piece>* pieces, int64_t stop_above = INT64_MAX) {
  const int64_t full = (budget - kSegmentCost) / kTile * kTile;   // budget >= 0
  if (full <= 0) return -1;
  if (pieces) pieces->clear();
  int64_t w = 0, room = budget, used = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = kv_indptr[b + 1] - kv_indptr[b];
    int64_t pos = 0;
    while (pos < n) {
      const int64_t rest = n - pos;
      if (room == budget && rest > full) {
        // fresh workers taking `full` tokens each until the rest fits one
        const int64_t k = (rest - 1) / full;
        if (pieces) {
          for (int64_t x = 0; x < k; ++x)
            pieces->push_back({w + x, b, static_cast<int32_t>(pos + x * full),
                               static_cast<int32_t>(pos + (x + 1) * full)});
        }
        w += k;
        pos += k * full;
        used = w;
        if (used > stop_above) return used;
        continue;
      }
      if (piece_cost(rest) <= room) {
        if (pieces) pieces->push_back({w, b, static_cast<int32_t>(pos), static_cast<int32_t>(n)});
        room -= piece_cost(rest);
        used = w + 1;
        pos = n;
        continue;
      }
      const int64_t take = room > kSegmentCost ? (room - kSegmentCost) / kTile * kTile : 0;
      if (take > 0) {
        if (pieces)
          pieces->push_back({w, b, static_cast<int32_t>(pos), static_cast<int32_t>(pos + take)});
        used = w + 1;
        pos += take;
      }
      ++w;
      room = budget;
      if (w > stop_above) return w;
    }
  }
  return used;
}

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

  int64_t limit;
  if (total == 0) {
    limit = 0;
  } else if (chunk_tokens > 0) {
    limit = cdiv(total, chunk_tokens);
  } else {
    // Short batches are latency-bound: each non-empty sequence may have a
    // worker of its own even when that leaves fewer than kMinWorkerTokens
    // tokens per worker.
    int64_t nonempty = 0;
    for (int32_t b = 0; b < batch; ++b) nonempty += kv_indptr[b + 1] > kv_indptr[b];
    limit = std::min<int64_t>(int64_t(num_cus) * kWorkersPerCu,
                              std::max(cdiv(total, kMinWorkerTokens), nonempty));
  }
  std::vector<Piece> pieces;
  pieces.reserve(static_cast<size_t>(batch) + static_cast<size_t>(std::max<int64_t>(limit, 0)) + 1);
  int64_t workers = 0;
  if (limit > 0) {
    // Smallest budget whose greedy fill needs at most `limit` workers. Every
    // cost is a multiple of kTile, so the fill depends on the budget only
    // through budget / kTile, and the smallest fitting budget is a multiple of
    // kTile: search over m = budget / kTile. Needing fewer workers as the
    // budget grows, the fill fits no m below the even share of the whole
    // sequences' costs (cuts only add cost), and the sum of those costs fits
    // one worker. Gallop up from the even share, then bisect.
    int64_t total_cost = 0;
    for (int32_t b = 0; b < batch; ++b) {
      const int64_t n = kv_indptr[b + 1] - kv_indptr[b];
      if (n > 0) total_cost += piece_cost(n);
    }
    const int64_t m_min = (kTile + kSegmentCost) / kTile;
    const int64_t m_max = std::max(m_min, total_cost / kTile);
    auto fits = [&](int64_t m) {
      const int64_t used = greedy_fill(kv_indptr, batch, m * kTile, nullptr, limit);
      return used >= 0 && used <= limit;
    };
    int64_t lo = std::min(m_max, std::max(m_min, cdiv(total_cost, kTile * limit)));
    int64_t hi = lo;
    for (int64_t step = 1; !fits(hi); step *= 2) {
      lo = hi + 1;
      hi = std::min(m_max, hi + step);
    }
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / 2;
      if (fits(mid)) hi = mid;
      else lo = mid + 1;
    }
    workers = greedy_fill(kv_indptr, batch, lo * kTile, &pieces);
  }
  p.n_workers = static_cast<int32_t>(workers);

  // The fill emits pieces in worker order, which is also sequence order, so
  // segments are written in one pass and grouped by worker already.
  p.segments.reserve(pieces.size());
  p.merges.reserve(static_cast<size_t>(batch));
  p.worker_ptr.assign(static_cast<size_t>(workers) + 1, 0);
  int32_t slot = 0;
  size_t i = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (kv_indptr[b + 1] == kv_indptr[b]) {
      p.merges.push_back({b, 0, 0, 0});
      continue;
    }
    size_t j = i;
    while (j < pieces.size() && pieces[j].b == b) ++j;
    const int32_t k = static_cast<int32_t>(j - i);
    for (size_t x = i; x < j; ++x) {
      p.segments.push_back(
          {b, pieces[x].lo, pieces[x].hi, k == 1 ? -1 : slot + static_cast<int32_t>(x - i)});
      ++p.worker_ptr[static_cast<size_t>(pieces[x].w) + 1];
    }
    if (k > 1) {
      p.merges.push_back({b, slot, k, 0});
      slot += k;
    }
    i = j;
  }
  for (size_t w = 1; w < p.worker_ptr.size(); ++w) p.worker_ptr[w] += p.worker_ptr[w - 1];
  p.n_slots = slot;
  *out = std::move(p);
  return true;
}

}  // namespace pkv
