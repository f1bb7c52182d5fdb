// Device-side helpers shared by the gfx950 kernels of libdg.
//
// Numeric conventions (the FP8 block-quantised GEMM page on lpnh.cn, s2.2,
// s3.1, s4.2): FP8 is E4M3 with bias 7, no infinities and largest finite value
// 448; rounding is to nearest, ties to even; BF16 outputs are rounded to
// nearest-even from FP32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Round a finite, non-negative binary32 magnitude to the nearest E4M3
// magnitude code (0x00..0x7E), ties to even, saturating at 448:
//  * a >= 448            -> 0x7E (448 is the largest finite E4M3 value and
//                           everything above it is nearer to 448 than to any
//                           other finite value)
//  * a <  2^-6           -> subnormal grid of 2^-9: code = RNE(a * 2^9),
//                           0..8 (8 is the smallest normal, code 0x08)
//  * otherwise           -> drop 20 significand bits with round-half-even;
//                           the carry into the exponent field is the binade
//                           step; rebias the exponent from 127 to 7.
// The caller ORs in the sign bit (0x80), so -0 and negative values that
// round to zero keep their sign.
__device__ __forceinline__ uint32_t e4m3_rne_mag(float mag) {
  const uint32_t a = __float_as_uint(mag);
  uint32_t code;
  if (a >= 0x43E00000u) {                 // 448.0f
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {           // 2^-6
    code = (uint32_t)__builtin_rintf(mag * 512.0f);
  } else {
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  }
  return code;
}

// Round-to-nearest-even FP32 -> BF16 bits for finite inputs.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float half_wave_max(float v) {
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace dg
