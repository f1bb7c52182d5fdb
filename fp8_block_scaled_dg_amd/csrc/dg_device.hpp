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
