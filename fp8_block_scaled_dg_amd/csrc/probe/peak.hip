// Measurement probe, not part of the GEMM library's C ABI: an FP8 MFMA loop
// that reports the dense FP8 matrix-core rate this GPU sustains, and the
// shader clock it ran at, so that results can be quoted against a measured
// peak as well as the published one.  Built as its own library
// (libdg_probe.so) and used only by the benchmark.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352dU; x ^= x >> 15; x *= 0x846ca68bU; x ^= x >> 16;
  return x;
}

// Eight independent accumulator chains per wave; operands are pseudo-random
// finite E4M3 codes (magnitude codes <= 0x7E with random signs), so the
// matrix cores switch like they do on quantised data.
__global__ void __launch_bounds__(256) mfma_fp8_loop(float* out, unsigned long long* clk, int iters) {
  const uint32_t tid = blockIdx.x * 256u + threadIdx.x;
  v8i a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t h = mix(tid * 16u + k), g = mix(tid * 16u + 8u + k);
    a[k] = (int)((h & 0x7E7E7E7Eu) | (g & 0x80808080u));
    b[k] = (int)((g & 0x7E7E7E7Eu) | (h & 0x80808080u));
  }
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  v4f c0 = z, c1 = z, c2 = z, c3 = z, c4 = z, c5 = z, c6 = z, c7 = z;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c0, 0, 0, 0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c1, 0, 0, 0, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c2, 0, 0, 0, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c3, 0, 0, 0, 0, 0, 0);
    c4 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c4, 0, 0, 0, 0, 0, 0);
    c5 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c5, 0, 0, 0, 0, 0, 0);
    c6 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c6, 0, 0, 0, 0, 0, 0);
    c7 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c7, 0, 0, 0, 0, 0, 0);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  const v4f t = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
  const float s = (t[0] + t[1]) + (t[2] + t[3]);
  out[tid] = s;
  if (tid == 0) {
    clk[0] = t1 - t0;  // shader clock cycles of this wave's loop
    clk[1] = r1 - r0;  // the same interval on the constant 100 MHz counter
  }
}

}  // namespace

extern "C" {

// Runs blocks x 256 threads, each wave issuing iters x 8 MFMAs of
// 16x16x128 FP8 (65536 FLOP each).  out: blocks*256 floats (device);
// clk: 2 uint64 (device).  Returns 0 or a HIP error code.
int dgp_mfma_fp8_loop(float* out, unsigned long long* clk, int blocks, int iters, void* stream) {
  if (!out || !clk || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(mfma_fp8_loop, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     out, clk, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
