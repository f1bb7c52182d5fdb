// FP8 E4M3 block quantiser for gfx950.
//
// Follows the quantisation recipe of the FP8 block-quantised GEMM page
// (lpnh.cn, s4.2; scale rule s3.1; all-zero blocks s5.4): for every block,
// amax = max|x|, s = amax / 448 as a binary32 division, then each element is
// divided by s in binary32 and rounded to the nearest E4M3 value, ties to even.
//
// HBM-bound streaming kernels (4 bytes in, 1 byte out per element, plus one
// FP32 scale per block).  Each thread keeps its slice of the block in
// registers, so the data is read from HBM exactly once: the amax reduction
// runs over registers (in-lane max, then cross-lane shuffles, then a short
// LDS exchange between waves for 128x128 blocks) before the encode pass.
//
// Division: x / s is computed as a correctly rounded binary32 quotient with
// one reciprocal per block and an FMA correction per element (Markstein's
// theorem: with r = RN(1/s) and q = RN(x r), q' = RN(q + (x - q s) r) is
// RN(x/s) when no intermediate underflows).  Underflowing quotients are below
// 2^-100 and encode to a signed zero whatever their low bits; blocks whose
// scale is itself subnormal fall back to the IEEE division sequence.
#include "dg_device.hpp"
#include "dg_internal.hpp"

namespace dg {

__device__ __forceinline__ float quotient_rn(float x, float s, float r) {
  const float q = x * r;
  const float e = __builtin_fmaf(-q, s, x);
  return __builtin_fmaf(e, r, q);
}

// |x| / s, correctly rounded, capped at 448.  The quotient is formed on |x|
// (s > 0, so |x/s| = |x|/s) and the sign bit is restored by the caller: the
// FMA correction would turn a -0 quotient into +0.  With a normal s the
// quotient never exceeds 448 by more than a few ulps, which rounds to 448
// anyway; with a subnormal s the scale itself may be off by a large factor
// and the quotient can exceed 448, where E4M3 rounding saturates to 448.
__device__ __forceinline__ float magnitude_quotient(float x, float s, float r, bool slow) {
  const float ax = fabsf(x);
  const float v = slow ? ax / s : quotient_rn(ax, s, r);
  return fminf(v, 448.0f);
}

// Sign bits of four values placed at bit 7 of each code byte.
__device__ __forceinline__ uint32_t zero_codes4(float4 v) {
  return ((__float_as_uint(v.x) >> 31) << 7) | ((__float_as_uint(v.y) >> 31) << 15) |
         ((__float_as_uint(v.z) >> 31) << 23) | ((__float_as_uint(v.w) >> 31) << 31);
}

// Round to the nearest E4M3 code, ties to even, with v_cvt_pk_fp8_f32 (OCP
// E4M3 on gfx950, default round-to-nearest-even mode).  Its result was
// compared on an MI355X with a ties-to-even encoder written from the E4M3
// field layout, for every binary32 magnitude below 464 and both signs
// (including binary32 subnormals and -0): no difference.
__device__ __forceinline__ uint32_t encode4(float4 v, float s, float r, bool slow) {
  int p = __builtin_amdgcn_cvt_pk_fp8_f32(magnitude_quotient(v.x, s, r, slow),
                                          magnitude_quotient(v.y, s, r, slow), 0, false);
  p = __builtin_amdgcn_cvt_pk_fp8_f32(magnitude_quotient(v.z, s, r, slow),
                                      magnitude_quotient(v.w, s, r, slow), p, true);
  return (uint32_t)p | zero_codes4(v);
}

__device__ __forceinline__ float abs_max4(float m, float4 v) {
  return fmaxf(fmaxf(m, fmaxf(fabsf(v.x), fabsf(v.y))), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// 128x128 blocks: one workgroup of 256 threads per block.  Thread t owns
// columns 4*(t%32) .. +3 of rows t/32 + 8*i, i = 0..15 (64 values).  A wave
// reads two full 512-byte row segments per instruction.
__global__ void __launch_bounds__(256)
quantize_block128_kernel(const float* __restrict__ x, uint8_t* __restrict__ q,
                         float* __restrict__ scales, int64_t rows, int64_t cols,
                         int64_t n_rb) {
  __shared__ float red[4];
  const int kb = blockIdx.x;
  const int64_t rb = blockIdx.y;
  const int t = threadIdx.x;
  const int64_t col = (int64_t)kb * 128 + 4 * (t & 31);
  const int64_t row0 = rb * 128 + (t >> 5);
  const bool col_ok = col < cols;

  float4 v[16];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t row = row0 + 8 * i;
    if (col_ok && row < rows)
      v[i] = *reinterpret_cast<const float4*>(x + row * cols + col);
    else
      v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    amax = abs_max4(amax, v[i]);
  }
  amax = wave_max(amax);
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  const float s = amax / 448.0f;
  if (t == 0) scales[(int64_t)kb * n_rb + rb] = s;
  const bool zero = (s == 0.0f);
  const bool slow = (s < 1.17549435e-38f);  // subnormal scale: 1/s may overflow
  const float r = zero ? 0.0f : 1.0f / s;
  if (!col_ok) return;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t row = row0 + 8 * i;
    if (row < rows) {
      const uint32_t packed = zero ? zero_codes4(v[i]) : encode4(v[i], s, r, slow);
      *reinterpret_cast<uint32_t*>(q + row * cols + col) = packed;
    }
  }
}

// 1x128 blocks (one scale per row per 128 columns): a 32-lane half-wave owns
// one (row, K-block); a workgroup of 256 threads covers 8 rows x RPT passes.
template <int RPT>
__global__ void __launch_bounds__(256)
quantize_row_kernel(const float* __restrict__ x, uint8_t* __restrict__ q,
                    float* __restrict__ scales, int64_t rows, int64_t cols) {
  const int kb = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t col = (int64_t)kb * 128 + 4 * (t & 31);
  const int64_t row0 = (int64_t)blockIdx.y * (8 * RPT) + (t >> 5);
  const bool col_ok = col < cols;

  float4 v[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int64_t row = row0 + 8 * i;
    if (col_ok && row < rows)
      v[i] = *reinterpret_cast<const float4*>(x + row * cols + col);
    else
      v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int64_t row = row0 + 8 * i;
    const float amax = half_wave_max(abs_max4(0.0f, v[i]));
    const float s = amax / 448.0f;
    if (row < rows) {
      if ((t & 31) == 0) scales[(int64_t)kb * rows + row] = s;
      if (col_ok) {
        const bool zero = (s == 0.0f);
        const bool slow = (s < 1.17549435e-38f);
        const float r = zero ? 0.0f : 1.0f / s;
        const uint32_t packed = zero ? zero_codes4(v[i]) : encode4(v[i], s, r, slow);
        *reinterpret_cast<uint32_t*>(q + row * cols + col) = packed;
      }
    }
  }
}

hipError_t launch_quantize(uint8_t* q, float* scales, const float* x, int64_t rows,
                           int64_t cols, int block_rows, hipStream_t stream) {
  const int64_t n_kb = (cols + 127) / 128;
  if (block_rows == 128) {
    const int64_t n_rb = (rows + 127) / 128;
    dim3 grid((unsigned)n_kb, (unsigned)n_rb);
    hipLaunchKernelGGL(quantize_block128_kernel, grid, dim3(256), 0, stream, x, q, scales,
                       rows, cols, n_rb);
  } else {
    constexpr int RPT = 4;
    const int64_t n_y = (rows + 8 * RPT - 1) / (8 * RPT);
    dim3 grid((unsigned)n_kb, (unsigned)n_y);
    hipLaunchKernelGGL(quantize_row_kernel<RPT>, grid, dim3(256), 0, stream, x, q, scales,
                       rows, cols);
  }
  return hipGetLastError();
}

}  // namespace dg
