// KV append for gfx950: store new K/V rows at slot positions of paged pools.
//
// What is stored follows the vLLM fork qsa.py page (_store_qsa_rows_kernel,
// qsa_store_cache_rows): row i goes to slot s = slot_mapping[i] of the pool,
// i.e. page s / page_size, position s % page_size; a slot outside
// [0, num_pages * page_size) stores nothing. Pools [P, page_size, Hkv, D]
// flatten to [P * page_size, Hkv * D], so the destination row is simply s.
//
// Design: pure data movement (HBM-bound, no arithmetic). One wave per row;
// lane l copies the 16-byte units l, l + 64, ... of the K row and of the V
// row, so every load and store of a wave covers up to 1 KB of contiguous
// bytes. Four rows per 256-thread workgroup.
#include <hip/hip_runtime.h>

#include "append.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowsPerBlock = 4;

__global__ __launch_bounds__(64 * kRowsPerBlock) void append_kernel(
    u32x4* __restrict__ k_pool, u32x4* __restrict__ v_pool, int64_t pool_slots,
    const u32x4* __restrict__ k_rows, const u32x4* __restrict__ v_rows,
    const int64_t* __restrict__ slot_mapping, int64_t n_rows, int32_t row_units) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const int64_t slot = slot_mapping[row];
  if (slot < 0 || slot >= pool_slots) return;
  const int lane = threadIdx.x & 63;
  const u32x4* ks = k_rows + row * row_units;
  const u32x4* vs = v_rows + row * row_units;
  u32x4* kd = k_pool + slot * row_units;
  u32x4* vd = v_pool + slot * row_units;
  for (int u = lane; u < row_units; u += 64) {
    const u32x4 kv = ks[u];
    const u32x4 vv = vs[u];
    kd[u] = kv;
    vd[u] = vv;
  }
}

}  // namespace

hipError_t launch_append(void* k_pool, void* v_pool, int64_t pool_slots, const void* k_rows,
                         const void* v_rows, const int64_t* slot_mapping, int64_t n_rows,
                         int32_t row_bytes, hipStream_t stream) {
  if (n_rows <= 0) return hipSuccess;
  const int64_t blocks = (n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(append_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(64 * kRowsPerBlock),
                     0, stream, static_cast<u32x4*>(k_pool), static_cast<u32x4*>(v_pool),
                     pool_slots, static_cast<const u32x4*>(k_rows),
                     static_cast<const u32x4*>(v_rows), slot_mapping, n_rows, row_bytes / 16);
  return hipGetLastError();
}

}  // namespace pkv
