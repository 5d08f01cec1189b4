// Device-side helpers shared by the HIP kernels of libspecattn (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// err_flags bits (mirrors include/specattn.h)
constexpr int kErrSlot = 1;
constexpr int kErrCapacity = 2;
constexpr int kErrToken = 4;
constexpr int kErrZeroResidual = 8;
constexpr int kErrTree = 16;

__device__ __forceinline__ void flag_error(int32_t* err, int bits) {
  if (err) atomicOr(err, bits);
}

// Cross-lane reductions over the four 16-lane groups of a wave: lane l and
// lanes l^16, l^32, l^48. v_permlane16_swap / v_permlane32_swap (called with
// the same register as both operands) return the pair {x[l], x[l^16]} (resp.
// l^32) in some order, so max / sum of the pair is the same on both partners
// and no LDS round trip is needed.
__device__ __forceinline__ float pair16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float group_max4(float x) { return pair32_max(pair16_max(x)); }
__device__ __forceinline__ float group_sum4(float x) { return pair32_sum(pair16_sum(x)); }

}  // namespace specattn
