// Kernel launchers of the paged-decode library (implemented in decode.hip and
// mla.hip). All pointers are device pointers; launches are asynchronous on
// `stream` and return the launch's hipError_t.
#ifndef PKV_KERNELS_H_
#define PKV_KERNELS_H_

#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace pkv {

// Paged GQA decode, Hq = 32, Hkv = 4, D = 128.
constexpr int kHq = 32;
constexpr int kHkv = 4;
constexpr int kHeadDim = 128;

// How the decode kernel finds the pool row (page * page_size + slot) of
// token t of sequence b:
// * CSR list (kv_indptr != NULL, page size 1): row = ids[kv_indptr[b] + t],
//   with kv_indptr[b] taken from the segment record (the plan's host copy);
// * block table (kv_indptr == NULL): row = (ids[b * table_stride + (t >> page_shift)]
//   << page_shift) | (t & (page_size - 1)).
struct KvAddressing {
  const int32_t* kv_indptr;
  const int32_t* ids;
  int64_t table_stride;
  int32_t page_shift;
};

// Where the first segment's ids start, for workers 0 .. kFirstArgWorkers - 1,
// passed in the kernel arguments: CSR (kv_indptr[b] + tok_begin, 0, n), block
// table (b, tok_begin, n), with n = tok_end - tok_begin (0 for a worker with
// no segment). Entries past the launch's worker count are never read.
constexpr int kFirstArgWorkers = 256;
struct FirstSegments {
  int32_t v[3 * kFirstArgWorkers];
};

// Which units do the decode kernel's two contractions (q.k scores and P.V):
// the matrix cores (v_mfma_f32_16x16x32_bf16, the 8 query heads of a KV head
// padded to 16 columns) or the vector ALU (v_dot2c_f32_bf16).
enum class DecodeEngine : int32_t { kMfma = 0, kDot2 = 1 };

// One workgroup per worker; worker w decodes the segments [s_begin, s_end)
// (start_event / stop_event: NULL, or events that take the kernel's own start
// and end times)
// named by its record workers[8w .. 8w+8) = (the first segment's five fields,
// s_begin, s_end, 0); segment records are 8 int32:
// (b, tok_begin, tok_end, slot, kv_indptr[b], 0, 0, 0).
hipError_t launch_decode_partial(const int32_t* workers, const int32_t* segments,
                                 const FirstSegments& firsts, int32_t n_workers,
                                 const uint16_t* q, const uint16_t* k_pool,
                                 const uint16_t* v_pool, const KvAddressing& addr,
                                 float sm_scale_log2, uint16_t* out, float* lse, float* part_o,
                                 float* part_lse, DecodeEngine engine, hipEvent_t start_event,
                                 hipEvent_t stop_event, hipStream_t stream);

// Merges the split sequences' partials: one workgroup per (merge record
// (b, first_slot, n_segments, 0), group of query heads). max_pieces is the
// largest n_segments of the records (it picks the kernel's shape);
// merges_host, a host copy of the records, lets up to 256 records travel in
// the kernel arguments (NULL: the kernel reads `merges`).
hipError_t launch_merge(const int32_t* merges, const int32_t* merges_host, int32_t n_merges,
                        int32_t max_pieces, const float* part_o, const float* part_lse,
                        uint16_t* out, float* lse, hipStream_t stream);

}  // namespace pkv

#endif  // PKV_KERNELS_H_
