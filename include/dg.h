/*
 * dg.h -- C ABI of the MI355X (gfx950) FP8 block-scaled GEMM library
 * (libdg.so).  C99-compatible; no HIP or PyTorch types appear here.
 *
 * The operations follow these public pages:
 *   [Q] "DeepGEMM ... FP8 block-quantised GEMM" (lpnh.cn/news/2826317)
 *   [D] "DeepGEMM: GPU high-efficiency BLAS kernel library" (pzsr.cn/news/21800)
 *   [M] "省算力新利器 DeepGEMM" (bjdmk.com.cn/news/5702840)
 *   [H] the DeepGEMM tuning walk-through on hotelren.com/news/5487494
 *
 * Conventions for every entry point
 *   - All data pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or retains them.  They must stay valid until the
 *     work queued on `stream` has finished.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream.  Calls are asynchronous and stream-ordered.
 *   - Arguments are validated on the host first.  On any error a non-zero
 *     status is returned and NOTHING is enqueued.  DG_ERR_HIP means a launch
 *     failed; faults inside a kernel surface at the caller's next
 *     synchronisation.
 *   - FP8 means E4M3 ("FN" encoding: bias 7, no infinities, S.1111.111 = NaN,
 *     largest finite 448) [Q s2.2, s3.1].  BF16 outputs are raw 16-bit
 *     patterns (uint16_t), rounded to nearest-even from FP32.
 *   - Scale arrays are FP32, K-block-major: the scale of row-block rb and
 *     K-block kb sits at scales[kb * n_row_blocks + rb] [Q s3.1: a separate
 *     array indexed by block, accessed contiguously].
 *   - Inputs must be finite.  Behaviour on NaN/Inf inputs is unspecified.
 *   - Split-K workspaces (the optional `workspace` argument of the small-M
 *     capable calls): the first DG_WORKSPACE_COUNTER_BYTES bytes hold one
 *     arrival counter per output tile and must be ZERO when a workspace is
 *     first used (allocate it zero-filled, or clear it once); every call
 *     leaves them zero again when its work completes, and no call ever
 *     writes anything else there, so one workspace can serve any sequence of
 *     calls, of any shape, that are ordered on the device.  The rest of the
 *     workspace need not be initialised and is clobbered.  Calls that may
 *     run at the same time (e.g. on different streams) need distinct
 *     workspaces; the library itself keeps no state between calls, so with
 *     distinct workspaces every call is re-entrant.
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DG_ABI_VERSION 3

/* Size of the arrival-counter region at the start of a split-K workspace. */
#define DG_WORKSPACE_COUNTER_BYTES 32768

enum {
    DG_OK = 0,
    DG_ERR_NULL = 1,        /* a required pointer is NULL                   */
    DG_ERR_SHAPE = 2,       /* a size is negative, zero or not a multiple   */
    DG_ERR_UNSUPPORTED = 3, /* block_rows / group count / epilogue unknown  */
    DG_ERR_ALIGN = 4,       /* a pointer is not suitably aligned            */
    DG_ERR_WORKSPACE = 5,   /* workspace given but smaller than required    */
    DG_ERR_HIP = 6,         /* the HIP runtime reported an error            */
    DG_ERR_SCRATCH = 7      /* shape needs more than the static scratch     */
};

/* ABI version of the loaded library (compare with DG_ABI_VERSION). */
int dg_abi_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char *dg_status_string(int status);

/* Row alignment each expert's group must be padded to in the grouped,
 * M-contiguous layout [D s3.3]: 128. */
int dg_get_mk_alignment_for_contiguous_layout(void);

/*
 * Block quantiser [Q s4.2 steps 1-5, s3.1, s5.4; D s4.1 to_fp8].
 *   x      : FP32 [rows][cols], row-major, 16-byte aligned.
 *   q      : out, E4M3 codes [rows][cols], same layout, 16-byte aligned.
 *   scales : out, FP32 [ceil(cols/128)][ceil(rows/block_rows)], 4-byte aligned.
 *   block_rows : 128 (128x128 blocks, weights) or 1 (1x128, per-row
 *            activation groups).  Edge blocks are clipped to the matrix.
 * For each block: amax = max|x|; s = amax / 448 (binary32 division);
 * s == 0 (all-zero block) gives codes +-0 with the element's sign; otherwise
 * q = round-to-nearest-even-E4M3(binary32(x / s)), saturating at 448.
 * Requirements: rows >= 1, cols >= 1, cols % 16 == 0; rows <= 65535 * 128
 * (block_rows 128) or 65535 * 32 (block_rows 1), else DG_ERR_SHAPE.
 */
int dg_quantize_fp8_block(uint8_t *q, float *scales, const float *x,
                          int64_t rows, int64_t cols, int block_rows, void *stream);

/*
 * Block quantiser with power-of-two (UE8M0) scales [D s3.1: the newer
 * architecture's scaling factors are UE8M0, four packed into one 32-bit
 * integer; Q s4.2 for the rest of the recipe].
 *   x, q, block_rows, requirements: as dg_quantize_fp8_block.
 *   sf : out, int32 [ceil(cols/512)][ceil(rows/block_rows)], 4-byte aligned:
 *        byte kb % 4 (least significant first) of word [kb / 4][rb] holds
 *        E for block (rb, kb); bytes past the last K block are written as 0.
 * For each block: t = amax / 448 (binary32 division, as in the FP32 recipe);
 * the scale is 2^(E - 127) with E the smallest value in [0, 254] such that
 * 2^(E - 127) >= t (t rounded up to a power of two, so no element exceeds
 * 448 after scaling; E = 0 for t < 2^-127, all-zero blocks included); then
 * q = round-to-nearest-even-E4M3(binary32(x / 2^(E - 127))), sign kept.
 */
int dg_quantize_fp8_block_ue8m0(uint8_t *q, int32_t *sf, const float *x,
                                int64_t rows, int64_t cols, int block_rows, void *stream);

/*
 * Workspace bytes dg_fp8_gemm_nt can use for split-K on this shape (0 when
 * the chosen plan needs none; otherwise DG_WORKSPACE_COUNTER_BYTES plus the
 * partial tiles).  Passing a smaller, non-NULL workspace is an error;
 * passing NULL/0 selects a plan that needs none.
 */
size_t dg_fp8_gemm_nt_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * NT GEMM with fine-grained block scaling [Q s2.2, s3.2; D s3.1, s4.1]:
 *   C[m][n] = bf16( sum_kb sa(m,kb) * sb(n,kb) * sum_{k in kb} A[m][k] * B[n][k] )
 * with FP32 accumulation and promotion once per 128-wide K block.
 *   c  : out, BF16 [M][N] row-major, 16-byte aligned.
 *   a  : E4M3 [M][K] row-major (K contiguous), 16-byte aligned.
 *   b  : E4M3 [N][K] row-major (K contiguous), 16-byte aligned.
 *   sa : FP32 [K/128][ceil(M/a_block_rows)], a_block_rows in {1, 128}.
 *   sb : FP32 [K/128][ceil(N/128)] (128x128 blocks).
 *   workspace / workspace_bytes: optional device scratch for split-K on
 *        small-M shapes (see dg_fp8_gemm_nt_workspace_bytes); may be NULL/0.
 *        16-byte aligned; its counter region must be zero on first use (see
 *        the conventions above); calls running at the same time need
 *        distinct workspaces.
 * Requirements: M >= 1; N >= 8, N % 8 == 0; K >= 128, K % 128 == 0;
 * M*K and N*K below 2^32 (byte offsets inside the kernels are 32-bit),
 * else DG_ERR_SHAPE.
 * The result is deterministic: a given plan sums in a fixed order.
 */
int dg_fp8_gemm_nt(uint16_t *c, const uint8_t *a, const uint8_t *b,
                   const float *sa, const float *sb, int a_block_rows,
                   int64_t M, int64_t N, int64_t K,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * NT GEMM with power-of-two (UE8M0) block scales [D s3.1; Q s2.2, s3.2]:
 *   C[m][n] = bf16( sum_kb 2^(Ea(m,kb) + Eb(n,kb) - 254) * sum_{k in kb} A[m][k] * B[n][k] )
 * with FP32 accumulation.  The scales are applied inside gfx950's scaled FP8
 * matrix instruction, so the sum runs in one FP32 accumulator per output
 * with no separate promotion step.
 *   c, a, b, a_block_rows, M, N, K and their requirements: as dg_fp8_gemm_nt.
 *   sfa : int32 [ceil(K/512)][ceil(M/a_block_rows)], packed as written by
 *         dg_quantize_fp8_block_ue8m0; sfb : int32 [ceil(K/512)][ceil(N/128)].
 *   workspace / workspace_bytes: optional split-K scratch for M <= 64, as
 *         for dg_fp8_gemm_nt (same size query, same workspace rules).
 * The kernel plan is dg_fp8_gemm_nt's (small-M kernels for M <= 64).
 * Deterministic.
 */
int dg_fp8_gemm_nt_ue8m0(uint16_t *c, const uint8_t *a, const uint8_t *b,
                         const int32_t *sfa, const int32_t *sfb, int a_block_rows,
                         int64_t M, int64_t N, int64_t K,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * NT GEMM of FP32 activations with FP8 weights, the activations quantised
 * inside the GEMM [Q s6: computing the scale factors inside the kernel saves
 * a round trip through global memory; s4.2 for the quantisation]:
 *   c  : out, BF16 [M][N] row-major, 16-byte aligned.
 *   a  : FP32 [M][K] row-major, 16-byte aligned (never written); for
 *        dg_fp8_gemm_nt_fused_a_bf16, BF16 bit patterns [M][K] (16-byte
 *        aligned), each widened exactly to FP32 before the quantisation.
 *   b  : E4M3 [N][K] row-major, 16-byte aligned; sb: FP32 [K/128][ceil(N/128)].
 * The codes and scales are the ones dg_quantize_fp8_block(a, block_rows = 1)
 * would write (for the BF16 form: of the widened values), formed on chip and
 * never stored; the product is then dg_fp8_gemm_nt's (a_block_rows = 1) of
 * those codes (bit for bit where both run the same kernel plan without split-K).
 *   workspace / workspace_bytes: optional split-K scratch, as for
 *        dg_fp8_gemm_nt (size from dg_fp8_gemm_nt_workspace_bytes(M, N, K);
 *        same workspace rules).
 * Requirements: 1 <= M <= DG_FUSED_A_MAX_M (small-batch decode); N >= 8,
 * N % 8 == 0; K >= 128, K % 128 == 0; N*K below 2^32; else DG_ERR_SHAPE.
 * Deterministic.
 */
#define DG_FUSED_A_MAX_M 64
int dg_fp8_gemm_nt_fused_a(uint16_t *c, const float *a, const uint8_t *b, const float *sb,
                           int64_t M, int64_t N, int64_t K,
                           void *workspace, size_t workspace_bytes, void *stream);
int dg_fp8_gemm_nt_fused_a_bf16(uint16_t *c, const uint16_t *a, const uint8_t *b,
                                const float *sb, int64_t M, int64_t N, int64_t K,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * NT GEMM with a fused epilogue [M s3.2: element-wise operators such as the
 * activation and the residual connection applied to the product while it is
 * still on chip, saving a write and a read of C; D s2.3: SwiGLU inside the
 * MoE kernel].  The product is dg_fp8_gemm_nt's FP32 accumulator acc; then,
 * in FP32, before the BF16 rounding:
 *   act = DG_EPI_NONE   v = acc
 *         DG_EPI_RELU   v = max(acc, 0)
 *         DG_EPI_SILU   v = acc / (1 + exp(-acc))
 *         DG_EPI_GELU   v = acc / 2 * (1 + erf(acc / sqrt(2)))
 *         DG_EPI_SWIGLU B's rows interleave gate and up (row 2j gate, row
 *                       2j+1 up): v[m][j] = silu(acc[m][2j]) * acc[m][2j+1],
 *                       so C has N/2 columns
 *   residual: optional BF16 [M][Nout] (Nout = N, or N/2 for SwiGLU),
 *             16-byte aligned, added to v; it may be c itself (in place:
 *             each element is read before it is written, by the same thread).
 *   c : out, BF16 [M][Nout].  Everything else as dg_fp8_gemm_nt.
 * An unknown act gives DG_ERR_UNSUPPORTED.  dg_fp8_gemm_nt is this call with
 * DG_EPI_NONE and no residual.
 */
enum {
    DG_EPI_NONE = 0,
    DG_EPI_RELU = 1,
    DG_EPI_SILU = 2,
    DG_EPI_GELU = 3,
    DG_EPI_SWIGLU = 4
};
int dg_fp8_gemm_nt_epilogue(uint16_t *c, const uint8_t *a, const uint8_t *b,
                            const float *sa, const float *sb, int a_block_rows,
                            int64_t M, int64_t N, int64_t K, int act, const uint16_t *residual,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Byte transpose of an FP8 (or any 1-byte) matrix [D s3.1: the TN, NN and
 * TT layouts take operands stored M- or N-major]:
 *   out[c][r] = in[r][c]; in [rows][cols], out [cols][rows], both 16-byte
 *   aligned, not overlapping (else DG_ERR_UNSUPPORTED).
 * Requirements: rows, cols >= 16 and multiples of 16; rows <= 65535 * 128.
 */
int dg_transpose_fp8(uint8_t *out, const uint8_t *in, int64_t rows, int64_t cols, void *stream);

/*
 * GEMM in any of the four operand layouts [D s3.1: NT, TN, NN, TT], with the
 * scales of dg_fp8_gemm_nt (they describe the logical blocks, whatever the
 * storage order):
 *   C[M][N] = A . B^T as in dg_fp8_gemm_nt, where
 *     layout DG_LAYOUT_NT: a [M][K], b [N][K]   (dg_fp8_gemm_nt itself)
 *            DG_LAYOUT_TN: a [K][M], b [K][N]
 *            DG_LAYOUT_NN: a [M][K], b [K][N]
 *            DG_LAYOUT_TT: a [K][M], b [N][K]
 * Operands stored M- or N-major are first transposed into the workspace
 * (dg_transpose_fp8), then the NT kernels run.  Workspace layout for TN, NN
 * and TT: the split-K region of dg_fp8_gemm_nt first (at least its
 * DG_WORKSPACE_COUNTER_BYTES counter region, zero on first use as for every
 * workspace, never written by the transposes), then the transposed copies.
 * dg_fp8_gemm_workspace_bytes(M, N, K, layout) is the full size (split-K
 * included when the small-M plan uses it); DG_WORKSPACE_COUNTER_BYTES plus
 * the transposed copies is the minimum (DG_ERR_WORKSPACE below that, with
 * nothing enqueued), which runs the plan without split-K.
 * Requirements: those of dg_fp8_gemm_nt; M % 16 == 0 when A is [K][M],
 * N % 16 == 0 when B is [K][N]; unknown layout -> DG_ERR_UNSUPPORTED.
 */
enum { DG_LAYOUT_NT = 0, DG_LAYOUT_TN = 1, DG_LAYOUT_NN = 2, DG_LAYOUT_TT = 3 };
size_t dg_fp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int layout);
int dg_fp8_gemm(uint16_t *c, const uint8_t *a, const uint8_t *b, const float *sa, const float *sb,
                int a_block_rows, int64_t M, int64_t N, int64_t K, int layout,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * K-grouped GEMM [D s3.2: grouped GEMM along the K axis, the MoE
 * weight-gradient layout]: group g covers K columns
 * [k_offsets[g], k_offsets[g+1]) and writes its own output
 *   C[g][m][n] = bf16( sum over the group's K blocks kb of
 *                      sa(m,kb) * sb(n,kb) * sum_{k in kb} A[m][k] * B[n][k] )
 *   a [M][K], b [N][K] (K-major; transpose first with dg_transpose_fp8),
 *   sa, sb over the whole K as in dg_fp8_gemm_nt,
 *   k_offsets : DEVICE int64 [num_groups + 1], 8-byte aligned, multiples of
 *               128 with 0 <= k_offsets[g] <= k_offsets[g+1] <= K (an empty
 *               group writes zeros; values outside the contract give
 *               unspecified results but no access outside the operands),
 *   c : out, BF16 [num_groups][M][N].
 * Requirements: those of dg_fp8_gemm_nt; num_groups >= 1.  Every shape runs
 * the 256 x 256 tile kernel.
 */
int dg_fp8_grouped_gemm_k(uint16_t *c, const uint8_t *a, const uint8_t *b, const float *sa,
                          const float *sb, int a_block_rows, const int64_t *k_offsets,
                          int num_groups, int64_t M, int64_t N, int64_t K, void *stream);

/*
 * Grouped GEMM, experts contiguous along M [D s2.3, s3.2, s3.3]:
 *   a         : E4M3 [M][K]; the rows of each expert are contiguous, experts
 *               in ascending id, each group padded to a multiple of 128 rows.
 *   b         : E4M3 [num_groups][N][K]; sb: FP32 [num_groups][K/128][ceil(N/128)].
 *   sa        : FP32 [K/128][ceil(M/a_block_rows)], a_block_rows in {1, 128}.
 *   m_indices : int32 [M]: expert id of each row, or -1 for a padding row.
 *               Within one 128-row block every row holds the same id or -1,
 *               and the block's first row holds the id (or the whole block
 *               is padding).
 *   c         : out, BF16 [M][N]; padding rows are written as zeros.
 * Row m computes C[m] = A[m] . B[g]^T with g = m_indices[m], scales as in
 * dg_fp8_gemm_nt using sb + g * (K/128) * ceil(N/128).
 * Requirements: M >= 128, M % 128 == 0; N >= 8, N % 8 == 0; K % 128 == 0;
 * 1 <= num_groups; M*K and N*K below 2^32.  Ids outside [-1, num_groups)
 * are a contract violation (a block whose first row holds one is written as
 * zeros; elsewhere the result is unspecified).
 */
int dg_fp8_grouped_gemm_contig(uint16_t *c, const uint8_t *a, const uint8_t *b,
                               const float *sa, const float *sb, int a_block_rows,
                               const int32_t *m_indices, int num_groups,
                               int64_t M, int64_t N, int64_t K, void *stream);

/*
 * dg_fp8_grouped_gemm_contig with the fused epilogue of dg_fp8_gemm_nt_epilogue
 * [M s3.2; D s2.3: SwiGLU inside the MoE kernel] applied to every real row:
 * act in DG_EPI_*, SwiGLU over interleaved gate/up rows of each expert's B
 * (C then has N/2 columns), optional BF16 residual [M][Nout] (16-byte
 * aligned, may be c).  Padding rows are written as zeros (no residual).
 * An unknown act gives DG_ERR_UNSUPPORTED; the rest as
 * dg_fp8_grouped_gemm_contig, which is this call with DG_EPI_NONE.
 */
int dg_fp8_grouped_gemm_contig_epilogue(uint16_t *c, const uint8_t *a, const uint8_t *b,
                                        const float *sa, const float *sb, int a_block_rows,
                                        const int32_t *m_indices, int num_groups, int64_t M,
                                        int64_t N, int64_t K, int act, const uint16_t *residual,
                                        void *stream);

/*
 * dg_fp8_grouped_gemm_contig_epilogue with the work shared out evenly over
 * the compute units [D s2.3, s3.2: the grouped MoE GEMM; H s5.6: persistent
 * workgroups that keep taking work instead of one per tile].  With one
 * workgroup per 256 x 256 output tile, a launch whose tiles are few next to
 * the compute units (or a little more than a multiple of them) leaves much
 * of the chip idle for part of the run.  Here one persistent workgroup per compute unit
 * takes an equal run of (tile, 128-wide K block) work; a tile split between
 * workgroups has each piece summed from zero in K order, the FP32 pieces
 * parked in the workspace, and the last piece to finish adds them in K order
 * and applies the epilogue.  The result is deterministic (the same bits on
 * every call for the same inputs and device) and within rounding of the
 * unsplit call's: the sums of the pieces associate differently.
 *   workspace / workspace_bytes: device scratch of at least
 *        dg_fp8_grouped_gemm_contig_workspace_bytes(M, N, K) bytes, 16-byte
 *        aligned, with the split-K workspace rules given at the top of this
 *        file (the counter region zero on first use and left zero).  NULL or
 *        0: this call is dg_fp8_grouped_gemm_contig_epilogue.  A smaller
 *        non-NULL workspace is DG_ERR_WORKSPACE.
 * Arguments, requirements and the other errors as
 * dg_fp8_grouped_gemm_contig_epilogue.  The query returns 0 for shapes the
 * call does not share out (more than 512 row blocks, more than 2048
 * possible tiles, or K above 2^20): those run one workgroup per tile,
 * workspace or not.  Measured on MI355X it pays where the matrix cores bound
 * the launch and the last wave of tiles is nearly empty; on MoE shapes bound
 * by streaming the expert weights the call without a workspace is faster.
 */
size_t dg_fp8_grouped_gemm_contig_workspace_bytes(int64_t M, int64_t N, int64_t K);
int dg_fp8_grouped_gemm_contig_balanced(uint16_t *c, const uint8_t *a, const uint8_t *b,
                                        const float *sa, const float *sb, int a_block_rows,
                                        const int32_t *m_indices, int num_groups, int64_t M,
                                        int64_t N, int64_t K, int act, const uint16_t *residual,
                                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * Grouped GEMM, experts contiguous along M, with power-of-two (UE8M0) block
 * scales [D s3.1: UE8M0 scales, four per int32; s2.3, s3.2, s3.3: grouped
 * MoE GEMM].  As dg_fp8_grouped_gemm_contig with the scale arrays of
 * dg_fp8_gemm_nt_ue8m0:
 *   sfa : int32 [ceil(K/512)][ceil(M/a_block_rows)];
 *   sfb : int32 [num_groups][ceil(K/512)][ceil(N/128)] (per expert as for the
 *         dense call).
 * Padding rows are written as zeros.  Requirements and errors as
 * dg_fp8_grouped_gemm_contig.  Deterministic.
 */
int dg_fp8_grouped_gemm_contig_ue8m0(uint16_t *c, const uint8_t *a, const uint8_t *b,
                                     const int32_t *sfa, const int32_t *sfb, int a_block_rows,
                                     const int32_t *m_indices, int num_groups, int64_t M,
                                     int64_t N, int64_t K, void *stream);

/*
 * Grouped GEMM, masked layout [D s2.3, s3.2: expert weights batched in one
 * grouped call].  The layout is a reading for decode-time MoE, where each
 * expert's token count is known only on the device: every expert has a fixed
 * capacity of max_m rows, and only the first masked_m[g] are computed.
 *   a        : E4M3 [num_groups][max_m][K].
 *   sa       : FP32 [num_groups][K/128][ceil(max_m/a_block_rows)], a_block_rows
 *              in {1, 128}.
 *   b        : E4M3 [num_groups][N][K]; sb: FP32 [num_groups][K/128][ceil(N/128)].
 *   masked_m : DEVICE int32 [num_groups], 4-byte aligned: valid rows of each
 *              group (values below 0 count as 0, above max_m as max_m).
 *   c        : out, BF16 [num_groups][max_m][N].  Rows m < masked_m[g] of
 *              group g get C[g][m] = A[g][m] . B[g]^T (scales as in
 *              dg_fp8_gemm_nt with the group's scale arrays); the other rows
 *              are not written.
 *   workspace: optional split-K scratch, as for dg_fp8_gemm_nt; its size is
 *              dg_fp8_grouped_gemm_masked_workspace_bytes (0: none needed);
 *              same workspace rules.
 * Requirements: those of dg_fp8_gemm_nt with M = max_m (max_m >= 1; N >= 8,
 * N % 8 == 0; K % 128 == 0; max_m*K and N*K below 2^32); 1 <= num_groups.
 * Rows are processed in chunks of up to 64 per workgroup, so B is streamed
 * once per chunk: the layout is meant for max_m <= 64.
 */
size_t dg_fp8_grouped_gemm_masked_workspace_bytes(int num_groups, int64_t max_m, int64_t N,
                                                  int64_t K);
int dg_fp8_grouped_gemm_masked(uint16_t *c, const uint8_t *a, const uint8_t *b,
                               const float *sa, const float *sb, int a_block_rows,
                               const int32_t *masked_m, int num_groups, int64_t max_m,
                               int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * dg_fp8_grouped_gemm_masked with the fused epilogue of
 * dg_fp8_gemm_nt_epilogue on the valid rows: act in DG_EPI_*, SwiGLU over
 * interleaved gate/up rows of each expert's B (C then [num_groups][max_m][N/2]),
 * optional BF16 residual laid out like C (16-byte aligned, may be c).  Rows
 * past masked_m[g] are not written.  dg_fp8_grouped_gemm_masked is this call
 * with DG_EPI_NONE and no residual.
 */
int dg_fp8_grouped_gemm_masked_epilogue(uint16_t *c, const uint8_t *a, const uint8_t *b,
                                        const float *sa, const float *sb, int a_block_rows,
                                        const int32_t *masked_m, int num_groups, int64_t max_m,
                                        int64_t N, int64_t K, int act, const uint16_t *residual,
                                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * dg_fp8_grouped_gemm_masked with power-of-two (UE8M0) block scales [D s3.1]:
 *   sfa : int32 [num_groups][ceil(K/512)][ceil(max_m/a_block_rows)];
 *   sfb : int32 [num_groups][ceil(K/512)][ceil(N/128)]
 * (each group's words as for dg_fp8_gemm_nt_ue8m0).  Everything else,
 * including the workspace size query, as dg_fp8_grouped_gemm_masked.
 */
int dg_fp8_grouped_gemm_masked_ue8m0(uint16_t *c, const uint8_t *a, const uint8_t *b,
                                     const int32_t *sfa, const int32_t *sfb, int a_block_rows,
                                     const int32_t *masked_m, int num_groups, int64_t max_m,
                                     int64_t N, int64_t K, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * dg_fp8_gemm_nt for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same operation, arguments (minus the workspace), requirements, kernel plan
 * and results, bit for bit, as dg_fp8_gemm_nt given a workspace of
 * dg_fp8_gemm_nt_workspace_bytes(M, N, K).  The split-K scratch (arrival
 * counters and partial tiles) is a static device array inside the library
 * instead: DG_NOALLOC_SCRATCH_BYTES on every GPU the library runs on, held
 * until the process ends.
 *   - Runs on the current device; a non-NULL stream must belong to it
 *     (DG_ERR_UNSUPPORTED otherwise).
 *   - A shape whose plan needs more than DG_NOALLOC_SCRATCH_BYTES of scratch
 *     gives DG_ERR_SCRATCH with nothing enqueued (the small-M plans need at
 *     most 8 MiB plus DG_WORKSPACE_COUNTER_BYTES, so none does today).
 *   - A call whose plan splits K first clears the counter region with a fill
 *     kernel on `stream`, then runs the GEMM; plans without split-K touch
 *     no scratch.
 *   - Every call on one GPU shares that GPU's array and leaves its contents
 *     behind: calls that may overlap on one GPU (different streams) race on
 *     it and must be ordered by the caller.
 *   - The first call on a device looks the array's device address up
 *     (hipGetSymbolAddress, with that device current) and keeps it.  No call
 *     allocates or frees memory.
 */
#define DG_NOALLOC_SCRATCH_BYTES (16u << 20)
int dg_fp8_gemm_nt_noalloc(uint16_t *c, const uint8_t *a, const uint8_t *b,
                           const float *sa, const float *sb, int a_block_rows,
                           int64_t M, int64_t N, int64_t K, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
