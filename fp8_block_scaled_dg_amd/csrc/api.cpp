// C ABI of libdg (declared in include/dg.h): host-side validation and
// dispatch to the gfx950 kernels.  Validation happens before any HIP call, so
// a rejected call enqueues nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "../../include/dg.h"
#include "dg_internal.hpp"

namespace {

static_assert(DG_WORKSPACE_COUNTER_BYTES == dg::kSplitkCounterBytes,
              "counter region of dg.h and of the kernels");

constexpr int64_t kMaxGridY = 65535;
constexpr int64_t kU32 = 4294967295LL;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int from_hip(hipError_t e) { return e == hipSuccess ? DG_OK : DG_ERR_HIP; }

// Checks shared by the dense and grouped GEMMs.
int check_gemm(const uint16_t* c, const uint8_t* a, const uint8_t* b, const float* sa,
               const float* sb, int a_block_rows, int64_t M, int64_t N, int64_t K) {
  if (!c || !a || !b || !sa || !sb) return DG_ERR_NULL;
  if (a_block_rows != 1 && a_block_rows != 128) return DG_ERR_UNSUPPORTED;
  if (M < 1 || N < 8 || K < 128) return DG_ERR_SHAPE;
  if (N % 8 != 0 || K % 128 != 0) return DG_ERR_SHAPE;
  // 32-bit tile offsets inside the kernels
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return DG_ERR_SHAPE;
  if (M * K > kU32 || N * K > kU32) return DG_ERR_SHAPE;
  if (!aligned(c, 16) || !aligned(a, 16) || !aligned(b, 16)) return DG_ERR_ALIGN;
  if (!aligned(sa, 4) || !aligned(sb, 4)) return DG_ERR_ALIGN;
  return DG_OK;
}

// A split-K workspace, when given, must hold what the small-M plan for this
// shape uses and be 16-byte aligned; a NULL pointer or a zero size means none.
int check_workspace(int64_t M, int64_t N, int64_t K, void** workspace, size_t* workspace_bytes) {
  if (*workspace != nullptr && *workspace_bytes > 0) {
    const size_t need = dg::skinny_applies(M, N, K) ? dg::skinny_workspace_bytes(M, N, K) : 0;
    if (*workspace_bytes < need) return DG_ERR_WORKSPACE;
    if (!aligned(*workspace, 16)) return DG_ERR_ALIGN;
  } else {
    *workspace = nullptr;  // one of the two missing: treat as "no workspace"
    *workspace_bytes = 0;
  }
  return DG_OK;
}

size_t align16(int64_t n) { return (size_t)((n + 15) / 16 * 16); }

// Workspace bytes for the operands a layout has to transpose.
size_t transpose_bytes(int64_t M, int64_t N, int64_t K, int layout) {
  const bool a_t = layout == DG_LAYOUT_TN || layout == DG_LAYOUT_TT;
  const bool b_n = layout == DG_LAYOUT_TN || layout == DG_LAYOUT_NN;
  return (a_t ? align16(M * K) : 0) + (b_n ? align16(N * K) : 0);
}

}  // namespace

extern "C" {

int dg_abi_version(void) { return DG_ABI_VERSION; }

const char* dg_status_string(int status) {
  switch (status) {
    case DG_OK: return "ok";
    case DG_ERR_NULL: return "a required pointer is NULL";
    case DG_ERR_SHAPE: return "invalid or unsupported shape";
    case DG_ERR_UNSUPPORTED: return "unsupported block_rows, group count or epilogue";
    case DG_ERR_ALIGN: return "pointer not suitably aligned";
    case DG_ERR_WORKSPACE: return "workspace smaller than required";
    case DG_ERR_HIP: return "HIP runtime error";
    case DG_ERR_SCRATCH: return "shape needs more split-K scratch than the static array holds";
    default: return "unknown status";
  }
}

int dg_get_mk_alignment_for_contiguous_layout(void) { return 128; }

int dg_quantize_fp8_block(uint8_t* q, float* scales, const float* x, int64_t rows, int64_t cols,
                          int block_rows, void* stream) {
  if (!q || !scales || !x) return DG_ERR_NULL;
  if (block_rows != 1 && block_rows != 128) return DG_ERR_UNSUPPORTED;
  if (rows < 1 || cols < 1 || cols % 16 != 0) return DG_ERR_SHAPE;
  const int64_t n_kb = (cols + 127) / 128;
  const int64_t grid_y = block_rows == 128 ? (rows + 127) / 128 : (rows + 31) / 32;
  if (grid_y > kMaxGridY || n_kb > INT32_MAX) return DG_ERR_SHAPE;
  if (rows > INT64_MAX / cols) return DG_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scales, 4)) return DG_ERR_ALIGN;
  return from_hip(dg::launch_quantize(q, scales, x, rows, cols, block_rows,
                                      static_cast<hipStream_t>(stream)));
}

int dg_quantize_fp8_block_ue8m0(uint8_t* q, int32_t* sf, const float* x, int64_t rows,
                                int64_t cols, int block_rows, void* stream) {
  if (!q || !sf || !x) return DG_ERR_NULL;
  if (block_rows != 1 && block_rows != 128) return DG_ERR_UNSUPPORTED;
  if (rows < 1 || cols < 1 || cols % 16 != 0) return DG_ERR_SHAPE;
  const int64_t n_kb = (cols + 127) / 128;
  const int64_t grid_y = block_rows == 128 ? (rows + 127) / 128 : (rows + 31) / 32;
  if (grid_y > kMaxGridY || n_kb > INT32_MAX) return DG_ERR_SHAPE;
  if (rows > INT64_MAX / cols) return DG_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(sf, 4)) return DG_ERR_ALIGN;
  return from_hip(dg::launch_quantize_ue8m0(q, reinterpret_cast<uint32_t*>(sf), x, rows, cols,
                                            block_rows, static_cast<hipStream_t>(stream)));
}

size_t dg_fp8_gemm_nt_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1) return 0;
  return dg::skinny_applies(M, N, K) ? dg::skinny_workspace_bytes(M, N, K) : 0;
}

int dg_fp8_gemm_nt(uint16_t* c, const uint8_t* a, const uint8_t* b, const float* sa,
                   const float* sb, int a_block_rows, int64_t M, int64_t N, int64_t K,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return dg_fp8_gemm_nt_epilogue(c, a, b, sa, sb, a_block_rows, M, N, K, DG_EPI_NONE, nullptr,
                                 workspace, workspace_bytes, stream);
}

int dg_fp8_gemm_nt_epilogue(uint16_t* c, const uint8_t* a, const uint8_t* b, const float* sa,
                            const float* sb, int a_block_rows, int64_t M, int64_t N, int64_t K,
                            int act, const uint16_t* residual, void* workspace,
                            size_t workspace_bytes, void* stream) {
  int st = check_gemm(c, a, b, sa, sb, a_block_rows, M, N, K);
  if (st != DG_OK) return st;
  if (act < DG_EPI_NONE || act > DG_EPI_SWIGLU) return DG_ERR_UNSUPPORTED;
  if (residual && !aligned(residual, 16)) return DG_ERR_ALIGN;
  const bool skinny = dg::skinny_applies(M, N, K);
  st = check_workspace(M, N, K, &workspace, &workspace_bytes);
  if (st != DG_OK) return st;
  dg::GemmProblem p{c, a, b, sa, sb, nullptr, 1, a_block_rows, M, N, K};
  p.epi.act = act;
  p.epi.res = residual;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (skinny) {
    if (dg::stream_preferred(M, N, K)) return from_hip(dg::launch_gemm_stream(p, s));
    return from_hip(dg::launch_gemm_skinny(p, workspace, workspace_bytes, s));
  }
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles > INT32_MAX) return DG_ERR_SHAPE;
  return from_hip(dg::launch_gemm_tiled(p, false, s));
}

int dg_fp8_gemm_nt_ue8m0(uint16_t* c, const uint8_t* a, const uint8_t* b, const int32_t* sfa,
                         const int32_t* sfb, int a_block_rows, int64_t M, int64_t N, int64_t K,
                         void* workspace, size_t workspace_bytes, void* stream) {
  // the FP32-scale checks apply unchanged (the scale pointers only need
  // 4-byte alignment in both forms)
  int st = check_gemm(c, a, b, reinterpret_cast<const float*>(sfa),
                      reinterpret_cast<const float*>(sfb), a_block_rows, M, N, K);
  if (st != DG_OK) return st;
  st = check_workspace(M, N, K, &workspace, &workspace_bytes);
  if (st != DG_OK) return st;
  dg::GemmProblem p{c, a, b, nullptr, nullptr, nullptr, 1, a_block_rows, M, N, K};
  p.sfa = reinterpret_cast<const uint32_t*>(sfa);
  p.sfb = reinterpret_cast<const uint32_t*>(sfb);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dg::skinny_applies(M, N, K)) {
    if (dg::stream_preferred(M, N, K)) return from_hip(dg::launch_gemm_stream(p, s));
    return from_hip(dg::launch_gemm_skinny(p, workspace, workspace_bytes, s));
  }
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles > INT32_MAX) return DG_ERR_SHAPE;
  return from_hip(dg::launch_gemm_tiled_ue8m0(p, s));
}

namespace {
int fused_a(uint16_t* c, const void* a, bool bf16, const uint8_t* b, const float* sb, int64_t M,
            int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  if (!c || !a || !b || !sb) return DG_ERR_NULL;
  if (M < 1 || M > DG_FUSED_A_MAX_M || N < 8 || K < 128) return DG_ERR_SHAPE;
  if (N % 8 != 0 || K % 128 != 0) return DG_ERR_SHAPE;
  if (N > INT32_MAX || K > INT32_MAX || N * K > kU32) return DG_ERR_SHAPE;
  if (!dg::skinny_applies(M, N, K)) return DG_ERR_SHAPE;
  if (!aligned(c, 16) || !aligned(a, 16) || !aligned(b, 16) || !aligned(sb, 4))
    return DG_ERR_ALIGN;
  const int st = check_workspace(M, N, K, &workspace, &workspace_bytes);
  if (st != DG_OK) return st;
  dg::GemmProblem p{c, nullptr, b, nullptr, sb, nullptr, 1, 1, M, N, K};
  return from_hip(dg::launch_gemm_skinny_fused_a(p, a, bf16, workspace, workspace_bytes,
                                                 static_cast<hipStream_t>(stream)));
}
}  // namespace

int dg_fp8_gemm_nt_fused_a(uint16_t* c, const float* a, const uint8_t* b, const float* sb,
                           int64_t M, int64_t N, int64_t K, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return fused_a(c, a, false, b, sb, M, N, K, workspace, workspace_bytes, stream);
}

int dg_fp8_gemm_nt_fused_a_bf16(uint16_t* c, const uint16_t* a, const uint8_t* b, const float* sb,
                                int64_t M, int64_t N, int64_t K, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return fused_a(c, a, true, b, sb, M, N, K, workspace, workspace_bytes, stream);
}

int dg_transpose_fp8(uint8_t* out, const uint8_t* in, int64_t rows, int64_t cols, void* stream) {
  if (!out || !in) return DG_ERR_NULL;
  if (rows < 16 || cols < 16 || rows % 16 != 0 || cols % 16 != 0) return DG_ERR_SHAPE;
  if ((rows + 127) / 128 > kMaxGridY || (cols + 127) / 128 > INT32_MAX) return DG_ERR_SHAPE;
  if (rows > INT64_MAX / cols) return DG_ERR_SHAPE;
  if (!aligned(out, 16) || !aligned(in, 16)) return DG_ERR_ALIGN;
  const uint8_t* o = out;
  if (o < in + rows * cols && in < o + rows * cols) return DG_ERR_UNSUPPORTED;  // overlap
  return from_hip(dg::launch_transpose_u8(out, in, rows, cols, static_cast<hipStream_t>(stream)));
}

size_t dg_fp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int layout) {
  if (M < 1 || N < 1 || K < 1 || layout < DG_LAYOUT_NT || layout > DG_LAYOUT_TT) return 0;
  const size_t nt = dg_fp8_gemm_nt_workspace_bytes(M, N, K);
  if (layout == DG_LAYOUT_NT) return nt;
  // split-K region (at least the counter region, which the transposes never
  // touch) first, then the transposed copies
  return (nt > DG_WORKSPACE_COUNTER_BYTES ? nt : DG_WORKSPACE_COUNTER_BYTES) +
         transpose_bytes(M, N, K, layout);
}

int dg_fp8_gemm(uint16_t* c, const uint8_t* a, const uint8_t* b, const float* sa, const float* sb,
                int a_block_rows, int64_t M, int64_t N, int64_t K, int layout, void* workspace,
                size_t workspace_bytes, void* stream) {
  if (layout < DG_LAYOUT_NT || layout > DG_LAYOUT_TT) return DG_ERR_UNSUPPORTED;
  if (layout == DG_LAYOUT_NT)
    return dg_fp8_gemm_nt(c, a, b, sa, sb, a_block_rows, M, N, K, workspace, workspace_bytes,
                          stream);
  // every check, the NT GEMM's included, before the first launch
  int st = check_gemm(c, a, b, sa, sb, a_block_rows, M, N, K);
  if (st != DG_OK) return st;
  const bool a_t = layout == DG_LAYOUT_TN || layout == DG_LAYOUT_TT;  // A given [K][M]
  const bool b_n = layout == DG_LAYOUT_TN || layout == DG_LAYOUT_NN;  // B given [K][N]
  if ((a_t && M % 16 != 0) || (b_n && N % 16 != 0)) return DG_ERR_SHAPE;
  if ((a_t && (K + 127) / 128 > kMaxGridY) || (b_n && (K + 127) / 128 > kMaxGridY))
    return DG_ERR_SHAPE;
  const bool skinny = dg::skinny_applies(M, N, K);
  if (!skinny && ((M + 255) / 256) * ((N + 255) / 256) > INT32_MAX) return DG_ERR_SHAPE;
  const size_t tb = transpose_bytes(M, N, K, layout);
  if (!workspace || workspace_bytes < DG_WORKSPACE_COUNTER_BYTES + tb) return DG_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return DG_ERR_ALIGN;
  // split-K when the workspace also holds the plan's partials after the
  // copies; otherwise the copies follow the (untouched) counter region
  const size_t split = skinny ? dg::skinny_workspace_bytes(M, N, K) : 0;
  const bool use_split = split > 0 && workspace_bytes >= split + tb;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  size_t used = use_split ? split : DG_WORKSPACE_COUNTER_BYTES;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* ak = a;
  const uint8_t* bk = b;
  if (a_t) {
    st = from_hip(dg::launch_transpose_u8(ws + used, a, K, M, s));  // [K][M] -> [M][K]
    if (st != DG_OK) return st;
    ak = ws + used;
    used += align16(M * K);
  }
  if (b_n) {
    st = from_hip(dg::launch_transpose_u8(ws + used, b, K, N, s));  // [K][N] -> [N][K]
    if (st != DG_OK) return st;
    bk = ws + used;
    used += align16(N * K);
  }
  return dg_fp8_gemm_nt(c, ak, bk, sa, sb, a_block_rows, M, N, K, use_split ? workspace : nullptr,
                        use_split ? split : 0, stream);
}

int dg_fp8_grouped_gemm_k(uint16_t* c, const uint8_t* a, const uint8_t* b, const float* sa,
                          const float* sb, int a_block_rows, const int64_t* k_offsets,
                          int num_groups, int64_t M, int64_t N, int64_t K, void* stream) {
  int st = check_gemm(c, a, b, sa, sb, a_block_rows, M, N, K);
  if (st != DG_OK) return st;
  if (!k_offsets) return DG_ERR_NULL;
  if (!aligned(k_offsets, 8)) return DG_ERR_ALIGN;
  if (num_groups < 1) return DG_ERR_UNSUPPORTED;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles * num_groups > INT32_MAX) return DG_ERR_SHAPE;
  if (M * N > INT64_MAX / num_groups) return DG_ERR_SHAPE;
  dg::GemmProblem p{c, a, b, sa, sb, nullptr, num_groups, a_block_rows, M, N, K};
  p.k_offsets = k_offsets;
  return from_hip(dg::launch_gemm_tiled_kgrouped(p, static_cast<hipStream_t>(stream)));
}

int dg_fp8_grouped_gemm_contig(uint16_t* c, const uint8_t* a, const uint8_t* b, const float* sa,
                               const float* sb, int a_block_rows, const int32_t* m_indices,
                               int num_groups, int64_t M, int64_t N, int64_t K, void* stream) {
  return dg_fp8_grouped_gemm_contig_epilogue(c, a, b, sa, sb, a_block_rows, m_indices, num_groups,
                                             M, N, K, DG_EPI_NONE, nullptr, stream);
}

int dg_fp8_grouped_gemm_contig_epilogue(uint16_t* c, const uint8_t* a, const uint8_t* b,
                                        const float* sa, const float* sb, int a_block_rows,
                                        const int32_t* m_indices, int num_groups, int64_t M,
                                        int64_t N, int64_t K, int act, const uint16_t* residual,
                                        void* stream) {
  return dg_fp8_grouped_gemm_contig_balanced(c, a, b, sa, sb, a_block_rows, m_indices, num_groups,
                                             M, N, K, act, residual, nullptr, 0, stream);
}

size_t dg_fp8_grouped_gemm_contig_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 128 || M % 128 != 0 || N < 8 || K < 128 || K % 128 != 0) return 0;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return 0;
  return dg::grouped_balanced_workspace_bytes(M, N, K);
}

int dg_fp8_grouped_gemm_contig_balanced(uint16_t* c, const uint8_t* a, const uint8_t* b,
                                        const float* sa, const float* sb, int a_block_rows,
                                        const int32_t* m_indices, int num_groups, int64_t M,
                                        int64_t N, int64_t K, int act, const uint16_t* residual,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_gemm(c, a, b, sa, sb, a_block_rows, M, N, K);
  if (st != DG_OK) return st;
  if (!m_indices) return DG_ERR_NULL;
  if (!aligned(m_indices, 4)) return DG_ERR_ALIGN;
  if (num_groups < 1) return DG_ERR_UNSUPPORTED;
  if (act < DG_EPI_NONE || act > DG_EPI_SWIGLU) return DG_ERR_UNSUPPORTED;
  if (residual && !aligned(residual, 16)) return DG_ERR_ALIGN;
  if (M % 128 != 0) return DG_ERR_SHAPE;
  if ((int64_t)num_groups * N * K / num_groups != N * K) return DG_ERR_SHAPE;
  if (workspace != nullptr && workspace_bytes > 0) {
    if (workspace_bytes < dg::grouped_balanced_workspace_bytes(M, N, K)) return DG_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return DG_ERR_ALIGN;
  } else {
    workspace = nullptr;  // one of the two missing: one workgroup per tile
    workspace_bytes = 0;
  }
  dg::GemmProblem p{c, a, b, sa, sb, m_indices, num_groups, a_block_rows, M, N, K};
  p.epi.act = act;
  p.epi.res = residual;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (!workspace) return from_hip(dg::launch_gemm_tiled(p, true, s));
  return from_hip(dg::launch_gemm_grouped_balanced(p, workspace, workspace_bytes, s));
}

int dg_fp8_grouped_gemm_contig_ue8m0(uint16_t* c, const uint8_t* a, const uint8_t* b,
                                     const int32_t* sfa, const int32_t* sfb, int a_block_rows,
                                     const int32_t* m_indices, int num_groups, int64_t M,
                                     int64_t N, int64_t K, void* stream) {
  int st = check_gemm(c, a, b, reinterpret_cast<const float*>(sfa),
                      reinterpret_cast<const float*>(sfb), a_block_rows, M, N, K);
  if (st != DG_OK) return st;
  if (!m_indices) return DG_ERR_NULL;
  if (!aligned(m_indices, 4)) return DG_ERR_ALIGN;
  if (num_groups < 1) return DG_ERR_UNSUPPORTED;
  if (M % 128 != 0) return DG_ERR_SHAPE;
  if ((int64_t)num_groups * N * K / num_groups != N * K) return DG_ERR_SHAPE;
  dg::GemmProblem p{c, a, b, nullptr, nullptr, m_indices, num_groups, a_block_rows, M, N, K};
  p.sfa = reinterpret_cast<const uint32_t*>(sfa);
  p.sfb = reinterpret_cast<const uint32_t*>(sfb);
  return from_hip(dg::launch_gemm_tiled_grouped_ue8m0(p, static_cast<hipStream_t>(stream)));
}

int dg_fp8_grouped_gemm_masked_ue8m0(uint16_t* c, const uint8_t* a, const uint8_t* b,
                                     const int32_t* sfa, const int32_t* sfb, int a_block_rows,
                                     const int32_t* masked_m, int num_groups, int64_t max_m,
                                     int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  int st = check_gemm(c, a, b, reinterpret_cast<const float*>(sfa),
                      reinterpret_cast<const float*>(sfb), a_block_rows, max_m, N, K);
  if (st != DG_OK) return st;
  if (!masked_m) return DG_ERR_NULL;
  if (!aligned(masked_m, 4)) return DG_ERR_ALIGN;
  if (num_groups < 1) return DG_ERR_UNSUPPORTED;
  if (max_m > INT64_MAX / K / num_groups || max_m > INT64_MAX / N / num_groups)
    return DG_ERR_SHAPE;
  if (dg::skinny_masked_grid(num_groups, max_m, N, K) > INT32_MAX) return DG_ERR_SHAPE;
  if (workspace != nullptr && workspace_bytes > 0) {
    if (workspace_bytes < dg::skinny_masked_workspace_bytes(num_groups, max_m, N, K))
      return DG_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return DG_ERR_ALIGN;
  } else {
    workspace = nullptr;
    workspace_bytes = 0;
  }
  dg::GemmProblem p{c, a, b, nullptr, nullptr, nullptr, num_groups, a_block_rows, max_m, N, K};
  p.sfa = reinterpret_cast<const uint32_t*>(sfa);
  p.sfb = reinterpret_cast<const uint32_t*>(sfb);
  return from_hip(dg::launch_gemm_skinny_masked(p, masked_m, max_m, workspace, workspace_bytes,
                                                static_cast<hipStream_t>(stream)));
}

size_t dg_fp8_grouped_gemm_masked_workspace_bytes(int num_groups, int64_t max_m, int64_t N,
                                                  int64_t K) {
  if (num_groups < 1 || max_m < 1 || N < 1 || K < 1) return 0;
  return dg::skinny_masked_workspace_bytes(num_groups, max_m, N, K);
}

int dg_fp8_grouped_gemm_masked(uint16_t* c, const uint8_t* a, const uint8_t* b, const float* sa,
                               const float* sb, int a_block_rows, const int32_t* masked_m,
                               int num_groups, int64_t max_m, int64_t N, int64_t K,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return dg_fp8_grouped_gemm_masked_epilogue(c, a, b, sa, sb, a_block_rows, masked_m, num_groups,
                                             max_m, N, K, DG_EPI_NONE, nullptr, workspace,
                                             workspace_bytes, stream);
}

int dg_fp8_grouped_gemm_masked_epilogue(uint16_t* c, const uint8_t* a, const uint8_t* b,
                                        const float* sa, const float* sb, int a_block_rows,
                                        const int32_t* masked_m, int num_groups, int64_t max_m,
                                        int64_t N, int64_t K, int act, const uint16_t* residual,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_gemm(c, a, b, sa, sb, a_block_rows, max_m, N, K);
  if (st != DG_OK) return st;
  if (!masked_m) return DG_ERR_NULL;
  if (!aligned(masked_m, 4)) return DG_ERR_ALIGN;
  if (num_groups < 1) return DG_ERR_UNSUPPORTED;
  if (act < DG_EPI_NONE || act > DG_EPI_SWIGLU) return DG_ERR_UNSUPPORTED;
  if (residual && !aligned(residual, 16)) return DG_ERR_ALIGN;
  if (max_m > INT64_MAX / K / num_groups || max_m > INT64_MAX / N / num_groups)
    return DG_ERR_SHAPE;
  if (dg::skinny_masked_grid(num_groups, max_m, N, K) > INT32_MAX) return DG_ERR_SHAPE;
  if (workspace != nullptr && workspace_bytes > 0) {
    if (workspace_bytes < dg::skinny_masked_workspace_bytes(num_groups, max_m, N, K))
      return DG_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return DG_ERR_ALIGN;
  } else {
    workspace = nullptr;
    workspace_bytes = 0;
  }
  dg::GemmProblem p{c, a, b, sa, sb, nullptr, num_groups, a_block_rows, max_m, N, K};
  p.epi.act = act;
  p.epi.res = residual;
  return from_hip(dg::launch_gemm_skinny_masked(p, masked_m, max_m, workspace, workspace_bytes,
                                                static_cast<hipStream_t>(stream)));
}

int dg_fp8_gemm_nt_noalloc(uint16_t* c, const uint8_t* a, const uint8_t* b, const float* sa,
                           const float* sb, int a_block_rows, int64_t M, int64_t N, int64_t K,
                           void* stream) {
  const int st = check_gemm(c, a, b, sa, sb, a_block_rows, M, N, K);
  if (st != DG_OK) return st;
  // plans that split K: the LDS-ring small-M kernel with a non-zero workspace
  const bool split = dg::skinny_applies(M, N, K) && !dg::stream_preferred(M, N, K) &&
                     dg::skinny_workspace_bytes(M, N, K) > 0;
  if (!split) return dg_fp8_gemm_nt(c, a, b, sa, sb, a_block_rows, M, N, K, nullptr, 0, stream);
  const size_t need = dg::skinny_workspace_bytes(M, N, K);
  if (need > DG_NOALLOC_SCRATCH_BYTES) return DG_ERR_SCRATCH;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return DG_ERR_HIP;
  if (s) {  // the scratch address is the current device's
    int sdev = 0;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess) return DG_ERR_HIP;
    if (sdev != cur) return DG_ERR_UNSUPPORTED;
  }
  void* ws = nullptr;
  if (dg::noalloc_scratch(&ws) != hipSuccess) return DG_ERR_HIP;
  const int zs = from_hip(dg::launch_zero_counters(ws, s));
  if (zs != DG_OK) return zs;
  return dg_fp8_gemm_nt(c, a, b, sa, sb, a_block_rows, M, N, K, ws, need, stream);
}

}  // extern "C"
