// Split-KV work partition for paged decode (host only, no HIP).
//
// A batch is cut into work items (b, tok_begin, tok_end, slot). Items of a
// sequence that fits one chunk write the final output (slot = -1); longer
// sequences are cut into equal tile-rounded chunks whose fp32 partials go to
// consecutive workspace slots and are combined by one merge record
// (b, first_slot, n_chunks, 0). The idea of splitting one row's keys into
// contiguous tiles with no empty split and merging by LSE is the vLLM fork
// qsa.py's (qsa_sparse_paged_attention); the chunk rule is this library's.
#ifndef PKV_PLAN_H_
#define PKV_PLAN_H_

#include <cstdint>
#include <string>
#include <vector>

namespace pkv {

constexpr int32_t kTile = 32;          // tokens per kernel tile; chunk lengths are multiples
constexpr int32_t kMinChunk = 256;     // shortest automatic chunk
constexpr int32_t kItemsPerCu = 2;     // automatic chunk aims at this many items per CU
constexpr int32_t kNoSplitChunk = 2147483647;

struct WorkItem {
  int32_t b, tok_begin, tok_end, slot;
};
struct MergeItem {
  int32_t b, first_slot, n_chunks, pad;
};

struct Partition {
  int32_t chunk = 0;
  int32_t n_slots = 0;
  int64_t total_tokens = 0;
  std::vector<WorkItem> items;
  std::vector<MergeItem> merges;
};

// Checks kv_indptr (starts at 0, non-decreasing, total < 2^31) and builds the
// partition. Returns false with a message in *err on bad input.
bool build_partition(const int32_t* kv_indptr, int32_t batch, int32_t num_cus,
                     bool allow_split, int32_t chunk_tokens, Partition* out, std::string* err);

}  // namespace pkv

#endif  // PKV_PLAN_H_
