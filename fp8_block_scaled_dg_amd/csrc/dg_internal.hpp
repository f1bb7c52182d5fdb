// Host-side declarations shared between the C ABI layer and the kernel
// launchers of libdg (internal; not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dg {

hipError_t launch_quantize(uint8_t* q, float* scales, const float* x, int64_t rows,
                           int64_t cols, int block_rows, hipStream_t stream);
// Power-of-two (UE8M0) scales, packed four K blocks per word:
// sf [ceil(cols/512)][ceil(rows/block_rows)].
hipError_t launch_quantize_ue8m0(uint8_t* q, uint32_t* sf, const float* x, int64_t rows,
                                 int64_t cols, int block_rows, hipStream_t stream);

// Fused epilogue of the BF16 write-back (bjdmk.com.cn DeepGEMM page, s3.2;
// SwiGLU per the pzsr.cn DeepGEMM page, s2.3).
enum EpiAct { EPI_NONE = 0, EPI_RELU = 1, EPI_SILU = 2, EPI_GELU = 3, EPI_SWIGLU = 4 };
struct Epilogue {
  int act = EPI_NONE;
  const uint16_t* res = nullptr;  // BF16 residual [M][ldc] (may be c itself), or null
  int64_t ldc = 0;                // C row length: N, or N / 2 for SwiGLU (0: N)
};

// out [cols][rows] = transpose of in [rows][cols] (bytes); rows, cols % 16 == 0.
hipError_t launch_transpose_u8(uint8_t* out, const uint8_t* in, int64_t rows, int64_t cols,
                               hipStream_t stream);

struct GemmProblem {
  uint16_t* c;
  const uint8_t* a;
  const uint8_t* b;
  const float* sa;
  const float* sb;
  const int32_t* m_indices;  // grouped only, else nullptr
  int num_groups;            // grouped only, else 1
  int a_block_rows;          // 1 or 128
  int64_t M, N, K;
  // power-of-two (UE8M0) scales, packed four K blocks per word, in place of
  // sa / sb (every kernel has a form that takes them), else nullptr
  const uint32_t* sfa = nullptr;
  const uint32_t* sfb = nullptr;
  Epilogue epi;
  // K-grouped (num_groups outputs, group g over K [k_offsets[g], k_offsets[g+1]))
  const int64_t* k_offsets = nullptr;
};

// The epilogue with its row length filled in.
inline Epilogue resolved_epilogue(const GemmProblem& q) {
  Epilogue e = q.epi;
  if (e.ldc == 0) e.ldc = e.act == EPI_SWIGLU ? q.N / 2 : q.N;
  return e;
}

// Large-tile MFMA kernel (dense or grouped).
hipError_t launch_gemm_tiled(const GemmProblem& p, bool grouped, hipStream_t stream);
// Grouped (M-contiguous) GEMM with the (tile, K block) work shared out
// evenly over one persistent workgroup per CU; pieces of split tiles are
// summed through the workspace (arrival counters, then partial tiles).  Falls
// back to launch_gemm_tiled without a large enough workspace or beyond the
// sizes it applies to.
bool grouped_balanced_applies(int64_t M, int64_t N, int64_t K);
size_t grouped_balanced_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_grouped_balanced(const GemmProblem& p, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream);
// Dense 256 x 256 tile kernel over K groups: C[g] = A[:, Kg] . B[:, Kg]^T.
hipError_t launch_gemm_tiled_kgrouped(const GemmProblem& p, hipStream_t stream);
// Dense 256 x 256 tile kernel with UE8M0 scales applied by the scaled MFMA.
hipError_t launch_gemm_tiled_ue8m0(const GemmProblem& p, hipStream_t stream);
// Grouped (M-contiguous) two-stage tile kernel with UE8M0 scales: sfa as
// dense, sfb [G][ceil(K/512)][ceil(N/128)].
hipError_t launch_gemm_tiled_grouped_ue8m0(const GemmProblem& p, hipStream_t stream);

// Split-K workspace of the small-M kernels: the first kSplitkCounterBytes
// hold one arrival counter per tile (zero on entry, left zero by every call),
// the partial tiles follow.  The region is the same for every shape, so one
// workspace can serve calls of any shape in turn.
constexpr size_t kSplitkCounterBytes = 32768;

// Skinny (small-M) kernel: workspace may be null (then no split-K).
size_t skinny_workspace_bytes(int64_t M, int64_t N, int64_t K);
bool skinny_applies(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_skinny(const GemmProblem& p, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);
// The same kernel with A given in FP32 or BF16 (M <= 64) and quantised with
// 1x128 blocks as it is staged; p.a and p.sa are unused.
hipError_t launch_gemm_skinny_fused_a(const GemmProblem& p, const void* af, bool bf16,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

// Masked grouped layout on the small-M ring kernel: A [G][max_m][K], C
// [G][max_m][N], masked_m[g] valid rows per group (device int32, clamped into
// [0, max_m]); p.M is unused, p.num_groups = G.  Workspace as for the plain
// call (null: no split-K); the grid size is checked against launch limits by
// the caller.
size_t skinny_masked_workspace_bytes(int num_groups, int64_t max_m, int64_t N, int64_t K);
int64_t skinny_masked_grid(int num_groups, int64_t max_m, int64_t N, int64_t K);
hipError_t launch_gemm_skinny_masked(const GemmProblem& p, const int32_t* masked_m, int64_t max_m,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

// Static scratch of dg_fp8_gemm_nt_noalloc: its device address on the
// current device (looked up once per device), and a kernel that zeroes its
// counter region.
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_zero_counters(void* scratch_ptr, hipStream_t stream);

// Streaming small-M kernel (no workspace), and whether it is the better of
// the two small-M kernels for a shape.
hipError_t launch_gemm_stream(const GemmProblem& p, hipStream_t stream);
bool stream_preferred(int64_t M, int64_t N, int64_t K);

}  // namespace dg
