// Internal helpers shared by the gfx950 kernels of libcsa (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bfloat16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// double -> bfloat16 bits with a single rounding (nearest, ties to even).
// The double is first narrowed to float with round-to-odd, which keeps enough
// information (24 >= 8 + 2 significant bits) for the final nearest-even step to
// equal a direct rounding of the double.
__device__ __forceinline__ uint16_t f64_to_bf16_bits(double v) {
  float f = static_cast<float>(v);
  double back = static_cast<double>(f);
  if (back != v) {
    uint32_t u = __float_as_uint(f);
    if (fabs(back) > fabs(v)) u -= 1u;  // truncate toward zero
    u |= 1u;                            // round to odd
    f = __uint_as_float(u);
  }
  return f32_to_bf16_bits(f);
}

// Largest b in [0, n) with cu[b] <= x, for non-decreasing cu with cu[0] <= x.
// With empty segments this picks the non-empty segment holding x.
__device__ __forceinline__ int segment_of(const int32_t* __restrict__ cu, int n, int x) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Order-preserving map float -> uint32 (larger float -> larger key); -0 ranks as +0.
__device__ __forceinline__ uint32_t float_order_key(float s) {
  s = s + 0.0f;  // -0.0 + 0.0 == +0.0 under round-to-nearest
  uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

}  // namespace csa
