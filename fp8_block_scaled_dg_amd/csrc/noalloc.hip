// Static split-K scratch for dg_fp8_gemm_nt_noalloc: callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation) get the small-M plan's workspace from a
// file-scope device array instead of an argument.
//
// The array exists once per GPU the library runs on and lives until the
// process ends.  In host code its name is only a host-side stand-in: the
// device address comes from hipGetSymbolAddress, called once per device
// with that device current, and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/dg.h"
#include "dg_internal.hpp"

namespace dg {
namespace {

static_assert(DG_NOALLOC_SCRATCH_BYTES > kSplitkCounterBytes, "scratch holds the counters");

__device__ __align__(256) uint8_t scratch[DG_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch`, per device (null: not yet)

// Zero the arrival counters (one int per tile) at the start of the scratch.
__global__ void __launch_bounds__(256) zero_counters_kernel(int4* p, int n4) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n4; i += gridDim.x * 256)
    p[i] = make_int4(0, 0, 0, 0);
}

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // this device is current
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

hipError_t launch_zero_counters(void* scratch_ptr, hipStream_t stream) {
  const int n4 = (int)(kSplitkCounterBytes / sizeof(int4));
  hipLaunchKernelGGL(zero_counters_kernel, dim3(8), dim3(256), 0, stream,
                     static_cast<int4*>(scratch_ptr), n4);
  return hipGetLastError();
}

}  // namespace dg
