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
// IEEE 754-2019 maximum (NaN propagates): v_maximum3_f32 on gfx950, with no
// quieting of its operands first, where fmaxf (NaN-ignoring) costs an extra
// v_max_f32 x, x, x per operand that the compiler cannot prove canonical.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float pair16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

// Lane moves inside 16-lane rows with DPP (a VALU operand modifier, no LDS
// round trip): xor 1 and xor 2 inside quads, the mirror of each 8-lane half
// (lane i <- 7 - i) and of each row (lane i <- 15 - i). After the xor steps
// every lane of a quad holds the quad's value; the mirrors then pair the two
// quads of a half and the two halves of a row.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_mov_dpp((int)(unsigned)b, CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(unsigned)(b >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

// Maximum over each 8-lane half row / each 16-lane row, in every lane of it.
__device__ __forceinline__ float half_row_max(float x) {
  x = fmaxf(x, dpp_f32<kDppXor1>(x));
  x = fmaxf(x, dpp_f32<kDppXor2>(x));
  return fmaxf(x, dpp_f32<kDppHalfMirror>(x));
}
__device__ __forceinline__ float row_max(float x) {
  return fmaxf(half_row_max(x), dpp_f32<kDppRowMirror>(half_row_max(x)));
}

// DPP move of a double where lanes without a source (or outside row_mask)
// read 0.0 instead.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64_or0(double x) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)b, CTRL, ROW_MASK, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(b >> 32), CTRL, ROW_MASK, 0xf, true);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

// Inclusive prefix sum of a double over the 64 lanes (lane order): shifts by
// 1, 2, 4, 8 inside each 16-lane row, then lane 15 of a row added to the next
// row (rows 1 and 3) and lane 31 to rows 2 and 3.
__device__ __forceinline__ double wave_scan_f64(double x) {
  x += dpp_f64_or0<0x111, 0xf>(x);  // row_shr:1
  x += dpp_f64_or0<0x112, 0xf>(x);  // row_shr:2
  x += dpp_f64_or0<0x114, 0xf>(x);  // row_shr:4
  x += dpp_f64_or0<0x118, 0xf>(x);  // row_shr:8
  x += dpp_f64_or0<0x142, 0xa>(x);  // row_bcast:15 into rows 1, 3
  x += dpp_f64_or0<0x143, 0xc>(x);  // row_bcast:31 into rows 2, 3
  return x;
}

// Sum of a double over the 64 lanes, the same value in every lane: pairs
// inside quads, halves and rows (DPP), then rows 16 and 32 apart
// (permlane swaps, each half of the double moved alike).
__device__ __forceinline__ double wave_sum_f64(double x) {
  x += dpp_f64<kDppXor1>(x);
  x += dpp_f64<kDppXor2>(x);
  x += dpp_f64<kDppHalfMirror>(x);
  x += dpp_f64<kDppRowMirror>(x);
  {
    const unsigned long long b = (unsigned long long)__double_as_longlong(x);
    const auto lo = __builtin_amdgcn_permlane16_swap((unsigned)b, (unsigned)b, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((unsigned)(b >> 32), (unsigned)(b >> 32), false, false);
    x = __longlong_as_double((long long)(((unsigned long long)hi[0] << 32) | lo[0])) +
        __longlong_as_double((long long)(((unsigned long long)hi[1] << 32) | lo[1]));
  }
  {
    const unsigned long long b = (unsigned long long)__double_as_longlong(x);
    const auto lo = __builtin_amdgcn_permlane32_swap((unsigned)b, (unsigned)b, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((unsigned)(b >> 32), (unsigned)(b >> 32), false, false);
    x = __longlong_as_double((long long)(((unsigned long long)hi[0] << 32) | lo[0])) +
        __longlong_as_double((long long)(((unsigned long long)hi[1] << 32) | lo[1]));
  }
  return x;
}

}  // namespace specattn
