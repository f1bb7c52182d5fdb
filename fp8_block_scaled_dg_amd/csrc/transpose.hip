// Byte transpose for FP8 operands given M- or N-major (the TN / NN / TT
// layouts of the DeepGEMM page on pzsr.cn, s3.1): out[c][r] = in[r][c].
//
// HBM-bound: every byte is read once and written once.  A workgroup of 256
// threads moves one 128 x 128-byte tile: 16-byte loads of whole row segments
// into LDS (row pitch 132 bytes, so the column reads below hit 64 different
// banks), then each thread gathers 64 bytes of one column and writes them as
// four 16-byte stores of one output row.  rows and cols are multiples of 16.
#include "dg_device.hpp"
#include "dg_internal.hpp"

namespace dg {
namespace {

constexpr int TT = 128;        // tile edge (bytes)
constexpr int PITCH = TT + 4;  // LDS row pitch

__global__ void __launch_bounds__(256)
transpose_u8_kernel(const uint8_t* __restrict__ in, uint8_t* __restrict__ out, int64_t rows,
                    int64_t cols) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[TT * PITCH];
  const int t = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * TT;
  const int64_t c0 = (int64_t)blockIdx.x * TT;
  // load: row (t / 8) + 32 i, 16 bytes at column 16 (t % 8)
  const int lc = 16 * (t & 7);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = (t >> 3) + 32 * i;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + lr < rows && c0 + lc < cols)
      v = *reinterpret_cast<const uint4*>(in + (r0 + lr) * cols + c0 + lc);
    uint32_t* d = reinterpret_cast<uint32_t*>(tile + lr * PITCH + lc);  // 4-byte aligned
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  }
  __syncthreads();
  // store: output row c0 + t / 2 holds input column t / 2; this thread covers
  // input rows 64 (t % 2) .. +63
  const int oc = t >> 1;
  const int h = (t & 1) * 64;
  if (c0 + oc >= cols) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rb = h + 16 * q;
    if (r0 + rb >= rows) break;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t x = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) x |= (uint32_t)tile[(rb + 4 * e + b) * PITCH + oc] << (8 * b);
      w[e] = x;
    }
    *reinterpret_cast<uint4*>(out + (c0 + oc) * rows + r0 + rb) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

hipError_t launch_transpose_u8(uint8_t* out, const uint8_t* in, int64_t rows, int64_t cols,
                               hipStream_t stream) {
  dim3 grid((unsigned)((cols + TT - 1) / TT), (unsigned)((rows + TT - 1) / TT));
  hipLaunchKernelGGL(transpose_u8_kernel, grid, dim3(256), 0, stream, in, out, rows, cols);
  return hipGetLastError();
}

}  // namespace dg
