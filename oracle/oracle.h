/*
 * Reference ("oracle") implementation of FP8 E4M3 block-scaled quantisation
 * and of the dequantised NT GEMM, on the CPU, in plain C.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this code; only the test suite, the smoke check and the CPU leg of
 * the benchmark use it.  It shares no code, header, table or constant with
 * the HIP kernels.
 *
 * Source pages (cited by title and section):
 *   "DeepGEMM ... FP8 block-quantised GEMM" (lpnh.cn/news/2826317):
 *     s2.2  128x128 blocks, one scale per block, E4M3 inputs, dequantise to
 *           FP32 and accumulate; product block scale = scale_a * scale_b
 *     s3.1  scale = max_abs / 448, stored as FP32 in a separate array
 *     s3.2  FP32 (never FP8) accumulation
 *     s4.2  the quantisation recipe: split into 128x128 blocks, take max_abs,
 *           scale = max_abs / 448.0, divide each element by its scale, round
 *           to the nearest FP8 value, preferring round-to-nearest-even
 *     s4.3  validate against an FP64 computation on the CPU
 *     s5.4  all-zero blocks need special handling (scale 0)
 *   "DeepGEMM: GPU high-efficiency BLAS kernel library" (pzsr.cn/news/21800):
 *     s3.1  NT layout (A not transposed, B transposed); SM90 FP32 scales;
 *           SM100 UE8M0 scales, four packed per 32-bit integer
 *     s3.2, s3.3  grouped GEMM along M for MoE, contiguous layout with an
 *           M alignment per group; grouping along K (weight gradients)
 *     s2.3  grouped GEMM batching the experts' weights (the masked,
 *           fixed-capacity decode layout is a reading of it)
 *     s4.1  to_fp8(a) -> (a_fp8, a_sf); fp8_gemm_nt(c, a, b, a_sf, b_sf)
 *
 * Parity status: every function here is pinned by the CPU tests (exhaustive
 * codec tables, a second independent encoder, exact-rational brute force on
 * tiny shapes, the PyTorch float8_e4m3fn cast, closed-form identities).
 */
#ifndef DG_ORACLE_H
#define DG_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* E4M3 ("FN": bias 7, no infinities, S.1111.111 is NaN, max 448). */
double  orc_e4m3_decode(uint8_t code);
/* Round-to-nearest-even encoder written from the exponent/mantissa fields. */
uint8_t orc_e4m3_encode_arith(float v);
/* Independent encoder: linear search over the 127 magnitudes with exact
 * midpoint comparisons. */
uint8_t orc_e4m3_encode_search(float v);

void orc_e4m3_encode_arith_n(const float *v, uint8_t *out, int64_t n);
void orc_e4m3_encode_search_n(const float *v, uint8_t *out, int64_t n);
void orc_e4m3_decode_n(const uint8_t *codes, double *out, int64_t n);

/* Block quantiser.  x: FP32 [rows][cols] row-major.  Blocks are
 * block_rows x 128 (block_rows in {1, 128}); edge blocks are clipped.
 * q: E4M3 codes [rows][cols].  scales: FP32 [ceil(cols/128)][ceil(rows/block_rows)]
 * (K-block-major).  Returns 0, or -1 on a bad argument / non-finite input. */
int orc_quantize_block(const float *x, int64_t rows, int64_t cols, int block_rows,
                       uint8_t *q, float *scales);

/* Block quantiser with power-of-two (UE8M0) scales: blocks as above;
 * exps: uint8 [ceil(cols/128)][ceil(rows/block_rows)], E with scale
 * 2^(E - 127) = t rounded up to a power of two, t = binary32(amax / 448)
 * (E = 0 when t < 2^-127, including all-zero blocks); q = RNE_E4M3(x / s). */
int orc_quantize_block_ue8m0(const float *x, int64_t rows, int64_t cols, int block_rows,
                             uint8_t *q, uint8_t *exps);
/* Pack exponents [n_kb][n_rb] four per word along K blocks:
 * packed [ceil(n_kb/4)][n_rb], byte kb % 4 of word [kb/4][rb]; unused bytes 0. */
void orc_ue8m0_pack(const uint8_t *exps, int64_t n_kb, int64_t n_rb, uint32_t *packed);

/* Per-tensor scaling (the baseline the block method is compared with): one
 * FP32 scale = amax(x) / 448 for the whole tensor, then the same division and
 * rounding.  Returns 0, or -1 on a bad argument / non-finite input. */
int orc_quantize_global(const float *x, int64_t rows, int64_t cols, uint8_t *q, float *scale);

/* Dequantised NT GEMM in FP64:
 * ref[m][n] = sum_kb (sa(m,kb) * sb(n,kb)) * sum_{k in kb} dec(qa[m][k]) dec(qb[n][k]).
 * qa [M][K], qb [N][K]; sa [ceil(K/128)][ceil(M/a_block_rows)];
 * sb [ceil(K/128)][ceil(N/128)]; ref [M][N]. */
int orc_gemm_nt(const uint8_t *qa, const float *sa, int a_block_rows,
                const uint8_t *qb, const float *sb,
                int64_t M, int64_t N, int64_t K, double *ref);

/* The same product at n_pts chosen (m, n) positions only. */
int orc_gemm_nt_points(const uint8_t *qa, const float *sa, int a_block_rows,
                       const uint8_t *qb, const float *sb,
                       int64_t M, int64_t N, int64_t K,
                       const int64_t *pm, const int64_t *pn, int64_t n_pts,
                       double *out);

/* Grouped, M-contiguous: row m uses expert g = m_indices[m] (B = qb + g*N*K,
 * sb + g*ceil(K/128)*ceil(N/128)); g == -1 marks a padding row whose output
 * row is zero.  rows_begin/rows_end restrict the rows computed (the rest of
 * ref is left untouched). */
int orc_grouped_gemm_contig(const uint8_t *qa, const float *sa, int a_block_rows,
                            const uint8_t *qb, const float *sb,
                            const int32_t *m_indices, int num_groups,
                            int64_t M, int64_t N, int64_t K,
                            int64_t rows_begin, int64_t rows_end, double *ref);

/* K-grouped product (pzsr.cn page s3.2): group g covers K columns
 * [k_offsets[g], k_offsets[g+1]) (multiples of 128, non-decreasing, within
 * K); out [G][M][N] = per-group dequantised A . B^T over that range, FP64.
 * A [M][K], B [N][K] K-major; scales as orc_gemm_nt over the whole K. */
/* Masked grouped layout: A [G][max_m][K], sa [G][K/128][ceil(max_m/a_block_rows)],
 * B [G][N][K], sb [G][K/128][ceil(N/128)], masked_m int32 [G] in [0, max_m];
 * ref [G][max_m][N]: rows m < masked_m[g] written, the others untouched. */
int orc_grouped_gemm_masked(const uint8_t *qa, const float *sa, int a_block_rows,
                            const uint8_t *qb, const float *sb, const int32_t *masked_m,
                            int num_groups, int64_t max_m, int64_t N, int64_t K, double *ref);
int orc_grouped_gemm_k(const uint8_t *qa, const float *sa, int a_block_rows,
                       const uint8_t *qb, const float *sb, const int64_t *k_offsets,
                       int num_groups, int64_t M, int64_t N, int64_t K, double *out);

/* Epilogue on an FP64 product acc [M][N] (bjdmk.com.cn page s3.2; pzsr.cn
 * page s2.3 for SwiGLU): act 0 none, 1 relu, 2 silu, 3 gelu (erf form),
 * 4 swiglu (B rows interleaved gate/up: out[m][j] = silu(acc[m][2j]) *
 * acc[m][2j+1], N/2 columns); then + residual (BF16 bits [M][Nout]) if not
 * NULL.  out: FP64 [M][Nout].  Returns 0, or -1 on a bad argument. */
int orc_epilogue(const double *acc, int64_t M, int64_t N, int act, const uint16_t *residual,
                 double *out);

#ifdef __cplusplus
}
#endif
#endif
