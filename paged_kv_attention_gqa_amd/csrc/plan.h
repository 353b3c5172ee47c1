// Split-KV work partition for paged decode (host only, no HIP).
//
// The batch's sequences, in order, are cut into contiguous pieces and dealt
// to workers (one workgroup of the decode kernel each) so that every worker
// gets about the same cost: a piece of n tokens costs its whole 32-token
// tiles plus kSegmentCost tokens for starting a segment (measured: a
// workgroup spends about half to one tile's time on each extra segment, and a
// ragged last tile nearly a whole tile's). Workers are filled greedily under a
// cost budget, the smallest budget that needs at most the allowed number of
// workers (a galloping search, then bisection); cuts inside a sequence fall on
// whole tiles. A worker's share is a list of segments
// (b, tok_begin, tok_end, slot), one per sequence it touches, with token
// positions relative to the sequence. A
// sequence that lies inside one worker is written directly (slot = -1); a
// sequence cut across workers leaves one normalised fp32 partial per segment
// in consecutive workspace slots, combined by a merge record
// (b, first_slot, n_segments, 0). Empty sequences get a merge record with no
// segments, which writes zeros and -inf. Splitting one row's keys into
// contiguous pieces with no empty piece and merging by LSE is the vLLM fork
// qsa.py's idea (qsa_sparse_paged_attention); the partition rule is this
// library's.
#ifndef PKV_PLAN_H_
#define PKV_PLAN_H_

#include <cstdint>
#include <string>
#include <vector>

namespace pkv {

constexpr int32_t kWorkersPerCu = 1;       // decode workgroups per CU
constexpr int32_t kMinWorkerTokens = 128;  // fewest tokens given to one worker
constexpr int32_t kTile = 32;              // tokens per decode tile
constexpr int32_t kSegmentCost = 32;       // tokens' worth of time to start a segment

struct Segment {
  int32_t b, tok_begin, tok_end, slot;
};
struct MergeItem {
  int32_t b, first_slot, n_segments, pad;
};

struct Partition {
  int32_t n_workers = 0;
  int32_t n_slots = 0;
  int64_t total_tokens = 0;
  std::vector<int32_t> worker_ptr;   // n_workers + 1 offsets into segments
  std::vector<Segment> segments;
  std::vector<MergeItem> merges;
};

// Checks kv_indptr (starts at 0, non-decreasing) and builds the partition.
// allow_split = false gives one worker per sequence. chunk_tokens > 0 sets
// the most workers to ceil(N / chunk_tokens); 0 to num_cus * kWorkersPerCu,
// or fewer for a short batch: max(ceil(N / kMinWorkerTokens), number of
// non-empty sequences). The fill may use fewer. Returns false with a message
// in *err on bad input.
bool build_partition(const int32_t* kv_indptr, int32_t batch, int32_t num_cus,
                     bool allow_split, int32_t chunk_tokens, Partition* out, std::string* err);

}  // namespace pkv

#endif  // PKV_PLAN_H_
