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

// One step of a sum that leaves different lanes with different results: lanes
// with bit 5 clear get a[i] + a[i | 32], lanes with it set b[i & ~32] + b[i]
// (v_permlane32_swap_b32 exchanges the upper half of its first operand with
// the lower half of its second). Eight values per lane reduce over the lane
// pair to four this way, with one exchange per pair of values.
__device__ __forceinline__ float split_sum_xor32(float a, float b) {
  const lane_u32x2 r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a),
                                                        __builtin_bit_cast(unsigned, b),
                                                        false, false);
  const unsigned x = r[0], y = r[1];
  return __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
}

// The same over lanes i and i ^ 16: lanes with bit 4 clear get a[i] +
// a[i | 16], lanes with it set b[i & ~16] + b[i].
__device__ __forceinline__ float split_sum_xor16(float a, float b) {
  const lane_u32x2 r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a),
                                                        __builtin_bit_cast(unsigned, b),
                                                        false, false);
  const unsigned x = r[0], y = r[1];
  return __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
}

// Lane i reads lane sel(i) of its own row of 16 through DPP (dpp_ctrl codes:
// quad permutations 0x00-0xff, row_mirror 0x140, row_half_mirror 0x141).
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xf, 0xf, false));
}

// Max and sum over the 16 lanes of a row (lanes 16k .. 16k + 15), the result
// in every lane of the row: exchanges with lane i ^ 1 and i ^ 2 (quad
// permutations), then with the mirrored lane of the half row and of the row,
// which after the quad steps holds the other quad's and the other half's value.
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_f32<0xb1>(x));    // quad_perm [1, 0, 3, 2]
  x = fmaxf(x, dpp_f32<0x4e>(x));    // quad_perm [2, 3, 0, 1]
  x = fmaxf(x, dpp_f32<0x141>(x));   // row_half_mirror
  return fmaxf(x, dpp_f32<0x140>(x));   // row_mirror
}

__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f32<0xb1>(x);
  x += dpp_f32<0x4e>(x);
  x += dpp_f32<0x141>(x);
  return x + dpp_f32<0x140>(x);
}

}  // namespace pkv

#endif  // PKV_LANES_H_
