// Cross-lane exchanges on the vector ALU for gfx950 wave64.
//
// v_permlane16_swap_b32 / v_permlane32_swap_b32 applied to two copies of a
// value leave every lane holding the pair (value of lane i with bit 4 / bit 5
// clear, value of lane i with it set) (checked on the GPU with an in-bounds
// probe), so a max or sum over lanes i and i ^ 16 (or i ^ 32) takes one VALU
// exchange instead of an LDS-routed ds_bpermute. The two halves of the pair
// are combined in the same order in every lane, so all lanes of the pair get
// bit-identical results. Each element of the returned pair is copied to a
// scalar before its bit cast (a bit cast applied directly to a vector element
// compiled as a cast of element 0).
#ifndef PKV_LANES_H_
#define PKV_LANES_H_

#include <hip/hip_runtime.h>

namespace pkv {

typedef unsigned int lane_u32x2 __attribute__((ext_vector_type(2)));

// (value of lane i & ~16, value of lane i | 16) in every lane i.
__device__ __forceinline__ lane_u32x2 pair_xor16(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  return __builtin_amdgcn_permlane16_swap(u, u, false, false);
}

// (value of lane i & ~32, value of lane i | 32) in every lane i.
__device__ __forceinline__ lane_u32x2 pair_xor32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  return __builtin_amdgcn_permlane32_swap(u, u, false, false);
}

__device__ __forceinline__ float max_xor16(float x) {
  const lane_u32x2 r = pair_xor16(x);
  const unsigned a = r[0], b = r[1];
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

__device__ __forceinline__ float max_xor32(float x) {
  const lane_u32x2 r = pair_xor32(x);
  const unsigned a = r[0], b = r[1];
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

__device__ __forceinline__ float sum_xor16(float x) {
  const lane_u32x2 r = pair_xor16(x);
  const unsigned a = r[0], b = r[1];
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

__device__ __forceinline__ float sum_xor32(float x) {
  const lane_u32x2 r = pair_xor32(x);
  const unsigned a = r[0], b = r[1];
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

}  // namespace pkv

#endif  // PKV_LANES_H_
