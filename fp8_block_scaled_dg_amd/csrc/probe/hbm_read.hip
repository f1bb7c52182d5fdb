// Measurement probe, not part of the GEMM library's C ABI: reads a [N][K]
// byte matrix from HBM the way the small-M GEMMs read their weights -- each
// wave owns 16 rows and a K range and loads 128 bytes of every row per K
// block, 8 KB per wave in flight, and nothing else (no A operand, no LDS, no
// arithmetic beyond folding the loaded words) -- so that the decode GEMMs
// can be compared with the rate a pure read of the same bytes reaches with
// the same number of workgroups.  Built into libdg_probe.so, used only by
// the benchmark.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

// Workgroup (tile, split) reads rows [64 tile, 64 tile + 64) (16 per wave)
// over K bytes [K split / S, K (split + 1) / S), 4 K blocks (4 x 2 KB per
// wave) per batch; the caller guarantees N % 64 == 0 and that every split's
// range is a multiple of 512 bytes.
__global__ void __launch_bounds__(256) hbm_read_kernel(const uint8_t* __restrict__ b, long K,
                                                       int splits, int* out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long tile = blockIdx.x / splits, split = blockIdx.x % splits;
  const long k0 = K * split / splits, k1 = K * (split + 1) / splits;
  const long row0 = tile * 64 + wave * 16;
  v4i acc = {0, 0, 0, 0};
  for (long k = k0; k + 512 <= k1; k += 512) {
    v4i v[8];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int idx = j * 64 + lane;  // row idx / 8, 16-byte chunk idx % 8
        v[s * 2 + j] = *reinterpret_cast<const v4i*>(b + (row0 + idx / 8) * K + k + s * 128 +
                                                      (idx % 8) * 16);
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc ^= v[i];
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

extern "C" {

// b: device [N][K] bytes; out: device int32 [N / 64 * splits * 256].
// Requirements (else returns 1, nothing launched): N >= 64, N % 64 == 0,
// splits >= 1, K % (512 * splits) == 0.  Returns 0 or a HIP error code.
int dgp_hbm_read(const void* b, long N, long K, int splits, int* out, void* stream) {
  if (!b || !out || N < 64 || N % 64 != 0 || splits < 1 || K % (512L * splits) != 0) return 1;
  const long grid = N / 64 * splits;
  if (grid > 0x7FFFFFFFL) return 1;
  hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(b), K, splits,
                     out);
  return (int)hipGetLastError();
}

}  // extern "C"
