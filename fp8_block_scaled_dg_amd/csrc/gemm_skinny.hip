// Small-M (decode) FP8 block-scaled NT GEMM for gfx950.  Not yet specialised:
// every shape currently runs on the tiled kernel.
#include "dg_device.hpp"
#include "dg_internal.hpp"

namespace dg {

bool skinny_applies(int64_t, int64_t, int64_t) { return false; }

size_t skinny_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_gemm_skinny(const GemmProblem&, void*, size_t, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace dg
