// KV append launcher (append.hip). Device pointers; asynchronous on `stream`.
#ifndef PKV_APPEND_H_
#define PKV_APPEND_H_

#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace pkv {

// Copies row i of k_rows / v_rows (row_bytes each, a multiple of 16) to row
// slot_mapping[i] of the flattened pools when 0 <= slot < pool_slots.
// Requires n_rows / 4 < 2^32 blocks.
hipError_t launch_append(void* k_pool, void* v_pool, int64_t pool_slots, const void* k_rows,
                         const void* v_rows, const int64_t* slot_mapping, int64_t n_rows,
                         int32_t row_bytes, hipStream_t stream);

}  // namespace pkv

#endif  // PKV_APPEND_H_
