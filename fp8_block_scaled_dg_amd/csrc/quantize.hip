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
// Division and rounding are the shared block encoder of dg_device.hpp: a
// correctly rounded binary32 quotient from one reciprocal per block and an
// FMA correction per element, rounded to E4M3 by the hardware conversion.
//
// The same kernels also produce power-of-two (UE8M0) scales (DeepGEMM page
// on pzsr.cn, s3.1): the FP32 scale amax / 448 rounded up to a power of two
// 2^(E - 127), stored as the byte E, four K blocks per 32-bit word.
#include "dg_device.hpp"
#include "dg_internal.hpp"

namespace dg {
namespace {

// The block's scale for the encoder, and its stored form: an FP32 scale at
// index [kb][rb] of a K-block-major array, or (E8) the UE8M0 exponent byte
// kb % 4 of the 32-bit word [kb / 4][rb]; the block that ends the K range
// also zeroes the word's bytes past it.
template <bool E8>
__device__ __forceinline__ BlockScale scale_and_store(float amax, void* scales, int64_t kb,
                                                      int64_t n_kb, int64_t n_rb, int64_t rb,
                                                      bool store) {
  if constexpr (E8) {
    const int e = ue8m0_exponent(amax / 448.0f);
    if (store) {
      uint8_t* w = static_cast<uint8_t*>(scales) + ((kb >> 2) * n_rb + rb) * 4;
      w[kb & 3] = (uint8_t)e;
      if (kb == n_kb - 1)
        for (int j = (int)(kb & 3) + 1; j < 4; ++j) w[j] = 0;
    }
    return pow2_block_scale(e);
  } else {
    const BlockScale bs = block_scale(amax);
    if (store) static_cast<float*>(scales)[kb * n_rb + rb] = bs.s;
    return bs;
  }
}

}  // namespace

// 128x128 blocks: one workgroup of 256 threads per block.  Thread t owns
// columns 4*(t%32) .. +3 of rows t/32 + 8*i, i = 0..15 (64 values).  A wave
// reads two full 512-byte row segments per instruction.
template <bool E8>
__global__ void __launch_bounds__(256)
quantize_block128_kernel(const float* __restrict__ x, uint8_t* __restrict__ q,
                         void* __restrict__ scales, int64_t rows, int64_t cols,
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

  const BlockScale bs = scale_and_store<E8>(amax, scales, kb, gridDim.x, n_rb, rb, t == 0);
  if (!col_ok) return;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t row = row0 + 8 * i;
    if (row < rows)
      *reinterpret_cast<uint32_t*>(q + row * cols + col) = encode4_block(v[i], bs);
  }
}

// 1x128 blocks (one scale per row per 128 columns): a 32-lane half-wave owns
// one (row, K-block); a workgroup of 256 threads covers 8 rows x RPT passes.
template <int RPT, bool E8>
__global__ void __launch_bounds__(256)
quantize_row_kernel(const float* __restrict__ x, uint8_t* __restrict__ q,
                    void* __restrict__ scales, int64_t rows, int64_t cols) {
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
    const BlockScale bs = scale_and_store<E8>(half_wave_max(abs_max4(0.0f, v[i])), scales, kb,
                                              gridDim.x, rows, row, row < rows && (t & 31) == 0);
    if (row < rows && col_ok)
      *reinterpret_cast<uint32_t*>(q + row * cols + col) = encode4_block(v[i], bs);
  }
}

namespace {

template <bool E8>
hipError_t launch_quantize_any(uint8_t* q, void* scales, const float* x, int64_t rows,
                               int64_t cols, int block_rows, hipStream_t stream) {
  const int64_t n_kb = (cols + 127) / 128;
  if (block_rows == 128) {
    const int64_t n_rb = (rows + 127) / 128;
    dim3 grid((unsigned)n_kb, (unsigned)n_rb);
    hipLaunchKernelGGL(quantize_block128_kernel<E8>, grid, dim3(256), 0, stream, x, q, scales,
                       rows, cols, n_rb);
  } else {
    constexpr int RPT = 4;
    const int64_t n_y = (rows + 8 * RPT - 1) / (8 * RPT);
    dim3 grid((unsigned)n_kb, (unsigned)n_y);
    hipLaunchKernelGGL((quantize_row_kernel<RPT, E8>), grid, dim3(256), 0, stream, x, q, scales,
                       rows, cols);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(uint8_t* q, float* scales, const float* x, int64_t rows,
                           int64_t cols, int block_rows, hipStream_t stream) {
  return launch_quantize_any<false>(q, scales, x, rows, cols, block_rows, stream);
}

hipError_t launch_quantize_ue8m0(uint8_t* q, uint32_t* sf, const float* x, int64_t rows,
                                 int64_t cols, int block_rows, hipStream_t stream) {
  return launch_quantize_any<true>(q, sf, x, rows, cols, block_rows, stream);
}

}  // namespace dg
