/*
 * CPU oracle for FP8 E4M3 block-scaled quantisation and the dequantised
 * NT GEMM.  TEST INFRASTRUCTURE ONLY: see oracle.h for the contract, the
 * pages followed, and who may use it.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math (x86-64 SSE: binary32 and
 * binary64 arithmetic with no excess precision).  Plain loops, no SIMD, no
 * BLAS, single thread.
 */
#include "oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* E4M3 codec.  The FP8 format is the E4M3 one with a largest finite value   */
/* of 448 ("DeepGEMM ... FP8 block-quantised GEMM", s2.2 and s3.1): four     */
/* exponent bits with bias 7, three mantissa bits, no infinities, and the    */
/* all-ones exponent+mantissa pattern reserved for NaN.                      */
/* ------------------------------------------------------------------------ */

double orc_e4m3_decode(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return sign ? -NAN : NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);           /* subnormal: m/8 * 2^(1-7) */
    else
        mag = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7)      */
    return sign ? -mag : mag;
}

/* Round a non-negative double that is an exact dyadic (no rounding happened
 * when it was formed) to the nearest integer, ties to even. */
static double rne_integer(double u)
{
    double f = floor(u);
    double frac = u - f; /* exact: u and f share the binade or f == 0 */
    if (frac > 0.5)
        return f + 1.0;
    if (frac < 0.5)
        return f;
    return fmod(f, 2.0) == 0.0 ? f : f + 1.0;
}

/* Encoder (i): work on the binary exponent and the significand directly.
 * Round-to-nearest-even ("... s4.2": nearest FP8 value, ties to even rather
 * than truncation).  Magnitudes past the largest finite value saturate to
 * 448 (a reading: the quantiser never produces them, see s3.1's scale rule);
 * the sign bit is always copied, so -0.0 and tiny negatives give 0x80. */
uint8_t orc_e4m3_encode_arith(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a;
    int ex;
    double u, n;
    if (isnan(v))
        return sign | 0x7F;
    a = fabs((double)v);
    if (a >= 448.0)
        return sign | 0x7E;
    if (a < 0.015625) { /* below the smallest normal, 2^-6: grid of 2^-9 */
        n = rne_integer(a * 512.0);             /* exact scaling by 2^9 */
        return sign | (uint8_t)n;               /* n == 8 is 2^-6, code 0x08 */
    }
    frexp(a, &ex);                              /* a = f * 2^ex, f in [0.5, 1) */
    ex -= 1;                                    /* a = g * 2^ex, g in [1, 2)  */
    u = ldexp(a, 3 - ex);                       /* significand in 1/8 units, [8, 16) */
    n = rne_integer(u);
    if (n == 16.0) {                            /* rounded up into the next binade */
        n = 8.0;
        ex += 1;
    }
    if (ex > 8 || (ex == 8 && n > 14.0))        /* beyond 448: saturate */
        return sign | 0x7E;
    return sign | (uint8_t)(((ex + 7) << 3) | ((int)n - 8));
}

/* Encoder (ii): a brute-force nearest search.  Code c (0..126) owns the open
 * interval between the midpoints to its neighbours; a magnitude on a
 * midpoint goes to the neighbour with an even code.  Midpoints of E4M3
 * magnitudes are exact doubles, so every comparison is exact. */
uint8_t orc_e4m3_encode_search(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a;
    int c;
    if (isnan(v))
        return sign | 0x7F;
    a = fabs((double)v);
    for (c = 0; c <= 126; ++c) {
        double val = orc_e4m3_decode((uint8_t)c);
        double lo = (c == 0) ? -1.0 : 0.5 * (orc_e4m3_decode((uint8_t)(c - 1)) + val);
        double hi = (c == 126) ? INFINITY : 0.5 * (val + orc_e4m3_decode((uint8_t)(c + 1)));
        if (a > lo && a < hi)
            return sign | (uint8_t)c;
        if (a == hi) /* tie between c and c + 1: take the even code */
            return sign | (uint8_t)((c % 2 == 0) ? c : c + 1);
    }
    return sign | 0x7E; /* not reached */
}

void orc_e4m3_encode_arith_n(const float *v, uint8_t *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = orc_e4m3_encode_arith(v[i]);
}

void orc_e4m3_encode_search_n(const float *v, uint8_t *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = orc_e4m3_encode_search(v[i]);
}

void orc_e4m3_decode_n(const uint8_t *codes, double *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = orc_e4m3_decode(codes[i]);
}

/* ------------------------------------------------------------------------ */
/* Quantiser ("... s4.2" steps 1-5, "... s3.1", "... s5.4").                */
/* ------------------------------------------------------------------------ */

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int orc_quantize_block(const float *x, int64_t rows, int64_t cols, int block_rows,
                       uint8_t *q, float *scales)
{
    int64_t n_rb, n_kb, rb, kb, r, k;
    if (!x || !q || !scales || rows < 0 || cols < 0)
        return -1;
    if (block_rows != 1 && block_rows != 128)
        return -1;
    for (r = 0; r < rows * cols; ++r)
        if (!isfinite(x[r]))
            return -1;
    n_rb = ceil_div(rows, block_rows);
    n_kb = ceil_div(cols, 128);
    for (rb = 0; rb < n_rb; ++rb) {
        int64_t r0 = rb * block_rows;
        int64_t r1 = r0 + block_rows < rows ? r0 + block_rows : rows;
        for (kb = 0; kb < n_kb; ++kb) {
            int64_t k0 = kb * 128;
            int64_t k1 = k0 + 128 < cols ? k0 + 128 : cols;
            float amax = 0.0f, s;
            /* step 2: the largest magnitude in the (clipped) block */
            for (r = r0; r < r1; ++r)
                for (k = k0; k < k1; ++k) {
                    float a = fabsf(x[r * cols + k]);
                    if (a > amax)
                        amax = a;
                }
            /* step 3: one binary32 division, stored as FP32 */
            s = amax / 448.0f;
            scales[kb * n_rb + rb] = s;
            /* step 4: divide by the scale in binary32, then round to E4M3 */
            for (r = r0; r < r1; ++r)
                for (k = k0; k < k1; ++k) {
                    float xv = x[r * cols + k];
                    if (s == 0.0f) {
                        q[r * cols + k] = signbit(xv) ? 0x80 : 0x00;
                    } else {
                        float v = xv / s;
                        q[r * cols + k] = orc_e4m3_encode_arith(v);
                    }
                }
        }
    }
    return 0;
}

/* Per-tensor ("global") scaling: the alternative that the block-wise method
 * is contrasted with on the bjdmk.com.cn DeepGEMM page (s3.3: one scaling
 * factor for the whole matrix instead of one per block).  The same steps as
 * the block quantiser with a single block covering the tensor: amax over all
 * elements, s = amax / 448 in binary32, v = x / s in binary32, E4M3 RNE. */
int orc_quantize_global(const float *x, int64_t rows, int64_t cols, uint8_t *q, float *scale)
{
    int64_t i, n;
    float amax = 0.0f, s;
    if (!x || !q || !scale || rows < 0 || cols < 0)
        return -1;
    n = rows * cols;
    for (i = 0; i < n; ++i) {
        float a;
        if (!isfinite(x[i]))
            return -1;
        a = fabsf(x[i]);
        if (a > amax)
            amax = a;
    }
    s = amax / 448.0f;
    *scale = s;
    for (i = 0; i < n; ++i) {
        if (s == 0.0f)
            q[i] = signbit(x[i]) ? 0x80 : 0x00;
        else
            q[i] = orc_e4m3_encode_arith(x[i] / s);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Power-of-two (UE8M0) block scales ("DeepGEMM: GPU high-efficiency BLAS    */
/* kernel library", s3.1: the newer architecture takes its scaling factors  */
/* as UE8M0, four packed into one 32-bit integer).  The pages do not say     */
/* how the power of two is chosen; the reading taken here keeps the FP32     */
/* recipe's guarantee that no element exceeds 448 after scaling: with        */
/* t = binary32(amax / 448) as before, s = 2^e with e the smallest integer   */
/* such that 2^e >= t, i.e. t rounded up to a power of two.  UE8M0 stores    */
/* E = e + 127 in one byte, 0..254 (255 is NaN); e below -127 (t == 0 or     */
/* t < 2^-127) is stored as E = 0.  Codes are RNE_E4M3(binary32(x / s)).     */
/* ------------------------------------------------------------------------ */

/* Smallest E in [0, 254] with 2^(E - 127) >= t, for finite t >= 0. */
static int ue8m0_exponent(float t)
{
    int ex, e;
    float f;
    if (t == 0.0f)
        return 0;
    f = frexpf(t, &ex);                 /* t = f * 2^ex, f in [0.5, 1) */
    e = (f == 0.5f) ? ex - 1 : ex;      /* ceil(log2 t) */
    e += 127;
    if (e < 0)
        e = 0;
    if (e > 254)
        e = 254;
    return e;
}

int orc_quantize_block_ue8m0(const float *x, int64_t rows, int64_t cols, int block_rows,
                             uint8_t *q, uint8_t *exps)
{
    int64_t n_rb, n_kb, rb, kb, r, k;
    if (!x || !q || !exps || rows < 0 || cols < 0)
        return -1;
    if (block_rows != 1 && block_rows != 128)
        return -1;
    for (r = 0; r < rows * cols; ++r)
        if (!isfinite(x[r]))
            return -1;
    n_rb = ceil_div(rows, block_rows);
    n_kb = ceil_div(cols, 128);
    for (rb = 0; rb < n_rb; ++rb) {
        int64_t r0 = rb * block_rows;
        int64_t r1 = r0 + block_rows < rows ? r0 + block_rows : rows;
        for (kb = 0; kb < n_kb; ++kb) {
            int64_t k0 = kb * 128;
            int64_t k1 = k0 + 128 < cols ? k0 + 128 : cols;
            float amax = 0.0f, s;
            int e;
            for (r = r0; r < r1; ++r)
                for (k = k0; k < k1; ++k) {
                    float a = fabsf(x[r * cols + k]);
                    if (a > amax)
                        amax = a;
                }
            e = ue8m0_exponent(amax / 448.0f);
            exps[kb * n_rb + rb] = (uint8_t)e;
            s = ldexpf(1.0f, e - 127);          /* exact, 2^-127 .. 2^127 */
            for (r = r0; r < r1; ++r)
                for (k = k0; k < k1; ++k)
                    q[r * cols + k] = orc_e4m3_encode_arith(x[r * cols + k] / s);
        }
    }
    return 0;
}

/* Four exponents per 32-bit word along the K-block index: word
 * [kb / 4][rb] holds the exponent of K block kb in byte kb % 4 (least
 * significant byte first); bytes past the last K block are 0. */
void orc_ue8m0_pack(const uint8_t *exps, int64_t n_kb, int64_t n_rb, uint32_t *packed)
{
    int64_t w, rb, j;
    for (w = 0; w < ceil_div(n_kb, 4); ++w)
        for (rb = 0; rb < n_rb; ++rb) {
            uint32_t v = 0;
            for (j = 0; j < 4; ++j) {
                int64_t kb = 4 * w + j;
                if (kb < n_kb)
                    v |= (uint32_t)exps[kb * n_rb + rb] << (8 * j);
            }
            packed[w * n_rb + rb] = v;
        }
}

/* ------------------------------------------------------------------------ */
/* Dequantised NT GEMM ("... s2.2", "... s3.2"; NT layout from "DeepGEMM:   */
/* GPU high-efficiency BLAS kernel library", s3.1 and s4.1).                 */
/* Within one 128-wide K block every product dec(a)*dec(b) is a multiple of  */
/* 2^-18 below 2^18, so the FP64 block sum is exact; the blocks are then     */
/* weighted by sa*sb (exact in FP64) and summed in ascending order.          */
/* ------------------------------------------------------------------------ */

static double dot_entry(const uint8_t *arow, const uint8_t *brow,
                        const float *sa, int64_t sa_stride, int64_t a_rb,
                        const float *sb, int64_t sb_stride, int64_t b_nb, int64_t K)
{
    int64_t n_kb = ceil_div(K, 128), kb, k;
    double total = 0.0;
    for (kb = 0; kb < n_kb; ++kb) {
        int64_t k0 = kb * 128;
        int64_t k1 = k0 + 128 < K ? k0 + 128 : K;
        double part = 0.0;
        double scale;
        for (k = k0; k < k1; ++k)
            part += orc_e4m3_decode(arow[k]) * orc_e4m3_decode(brow[k]);
        scale = (double)sa[kb * sa_stride + a_rb] * (double)sb[kb * sb_stride + b_nb];
        total += scale * part;
    }
    return total;
}

static int check_gemm_args(const uint8_t *qa, const float *sa, int a_block_rows,
                           const uint8_t *qb, const float *sb,
                           int64_t M, int64_t N, int64_t K)
{
    if (!qa || !sa || !qb || !sb || M < 0 || N < 0 || K < 0)
        return -1;
    if (a_block_rows != 1 && a_block_rows != 128)
        return -1;
    return 0;
}

int orc_gemm_nt(const uint8_t *qa, const float *sa, int a_block_rows,
                const uint8_t *qb, const float *sb,
                int64_t M, int64_t N, int64_t K, double *ref)
{
    int64_t m, n, sa_stride, sb_stride;
    if (check_gemm_args(qa, sa, a_block_rows, qb, sb, M, N, K) || !ref)
        return -1;
    sa_stride = ceil_div(M, a_block_rows);
    sb_stride = ceil_div(N, 128);
    for (m = 0; m < M; ++m)
        for (n = 0; n < N; ++n)
            ref[m * N + n] = dot_entry(qa + m * K, qb + n * K, sa, sa_stride,
                                       m / a_block_rows, sb, sb_stride, n / 128, K);
    return 0;
}

int orc_gemm_nt_points(const uint8_t *qa, const float *sa, int a_block_rows,
                       const uint8_t *qb, const float *sb,
                       int64_t M, int64_t N, int64_t K,
                       const int64_t *pm, const int64_t *pn, int64_t n_pts,
                       double *out)
{
    int64_t i, sa_stride, sb_stride;
    if (check_gemm_args(qa, sa, a_block_rows, qb, sb, M, N, K) || !pm || !pn || !out)
        return -1;
    sa_stride = ceil_div(M, a_block_rows);
    sb_stride = ceil_div(N, 128);
    for (i = 0; i < n_pts; ++i) {
        int64_t m = pm[i], n = pn[i];
        if (m < 0 || m >= M || n < 0 || n >= N)
            return -1;
        out[i] = dot_entry(qa + m * K, qb + n * K, sa, sa_stride, m / a_block_rows,
                           sb, sb_stride, n / 128, K);
    }
    return 0;
}

/* Grouped GEMM with experts' rows concatenated along M ("DeepGEMM: GPU
 * high-efficiency BLAS kernel library", s2.3, s3.2, s3.3). */
int orc_grouped_gemm_contig(const uint8_t *qa, const float *sa, int a_block_rows,
                            const uint8_t *qb, const float *sb,
                            const int32_t *m_indices, int num_groups,
                            int64_t M, int64_t N, int64_t K,
                            int64_t rows_begin, int64_t rows_end, double *ref)
{
    int64_t m, n, sa_stride, n_nb, n_kb;
    if (check_gemm_args(qa, sa, a_block_rows, qb, sb, M, N, K) || !m_indices || !ref)
        return -1;
    if (rows_begin < 0 || rows_end > M || rows_begin > rows_end || num_groups < 1)
        return -1;
    sa_stride = ceil_div(M, a_block_rows);
    n_nb = ceil_div(N, 128);
    n_kb = ceil_div(K, 128);
    for (m = rows_begin; m < rows_end; ++m) {
        int32_t g = m_indices[m];
        if (g < -1 || g >= num_groups)
            return -1;
        for (n = 0; n < N; ++n) {
            if (g < 0) {
                ref[m * N + n] = 0.0;
                continue;
            }
            ref[m * N + n] = dot_entry(qa + m * K, qb + (int64_t)g * N * K + n * K,
                                       sa, sa_stride, m / a_block_rows,
                                       sb + (int64_t)g * n_kb * n_nb, n_nb, n / 128, K);
        }
    }
    return 0;
}

/* Masked grouped GEMM ("DeepGEMM: GPU high-efficiency BLAS kernel library", */
/* s2.3 and s3.2: expert weights batched in one grouped call; the layout is  */
/* the decode-time one, where each expert's row count is known only on the   */
/* device): group g owns a fixed capacity of max_m rows of A and C, of which */
/* the first masked_m[g] are valid.  ref[g][m] = A[g][m] . B[g]^T with the   */
/* group's scales for m < masked_m[g]; the other rows of ref are not written */
/* (the caller pre-fills them).  masked_m[g] must lie in [0, max_m].          */
int orc_grouped_gemm_masked(const uint8_t *qa, const float *sa, int a_block_rows,
                            const uint8_t *qb, const float *sb, const int32_t *masked_m,
                            int num_groups, int64_t max_m, int64_t N, int64_t K, double *ref)
{
    int64_t g, m, n, sa_stride, n_nb, n_kb;
    if (check_gemm_args(qa, sa, a_block_rows, qb, sb, max_m, N, K) || !masked_m || !ref ||
        num_groups < 1)
        return -1;
    sa_stride = ceil_div(max_m, a_block_rows);
    n_nb = ceil_div(N, 128);
    n_kb = ceil_div(K, 128);
    for (g = 0; g < num_groups; ++g) {
        const uint8_t *ag = qa + g * max_m * K;
        const float *sag = sa + g * n_kb * sa_stride;
        const uint8_t *bg = qb + g * N * K;
        const float *sbg = sb + g * n_kb * n_nb;
        if (masked_m[g] < 0 || masked_m[g] > max_m)
            return -1;
        for (m = 0; m < masked_m[g]; ++m)
            for (n = 0; n < N; ++n)
                ref[(g * max_m + m) * N + n] =
                    dot_entry(ag + m * K, bg + n * K, sag, sa_stride, m / a_block_rows,
                              sbg, n_nb, n / 128, K);
    }
    return 0;
}

/* K-grouped GEMM ("DeepGEMM: GPU high-efficiency BLAS kernel library",     */
/* s3.2: grouped GEMM along the K axis, for MoE weight gradients): group g  */
/* owns the K range [k_offsets[g], k_offsets[g+1]) (multiples of 128) and    */
/* out[g] = A[:, range] . B[:, range]^T, with the scales of those K blocks.  */
int orc_grouped_gemm_k(const uint8_t *qa, const float *sa, int a_block_rows,
                       const uint8_t *qb, const float *sb, const int64_t *k_offsets,
                       int num_groups, int64_t M, int64_t N, int64_t K, double *out)
{
    int64_t g, m, n, sa_stride, sb_stride;
    if (check_gemm_args(qa, sa, a_block_rows, qb, sb, M, N, K) || !k_offsets || !out ||
        num_groups < 1)
        return -1;
    sa_stride = ceil_div(M, a_block_rows);
    sb_stride = ceil_div(N, 128);
    for (g = 0; g < num_groups; ++g) {
        int64_t k0 = k_offsets[g], k1 = k_offsets[g + 1];
        if (k0 < 0 || k1 < k0 || k1 > K || k0 % 128 != 0 || k1 % 128 != 0)
            return -1;
        for (m = 0; m < M; ++m)
            for (n = 0; n < N; ++n) {
                double total = 0.0;
                int64_t kb;
                for (kb = k0 / 128; kb < k1 / 128; ++kb) {
                    double part = 0.0;
                    int64_t k;
                    for (k = kb * 128; k < kb * 128 + 128; ++k)
                        part += orc_e4m3_decode(qa[m * K + k]) * orc_e4m3_decode(qb[n * K + k]);
                    total += (double)sa[kb * sa_stride + m / a_block_rows] *
                             (double)sb[kb * sb_stride + n / 128] * part;
                }
                out[(g * M + m) * N + n] = total;
            }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Epilogue fused into the GEMM's write-back ("省算力新利器 DeepGEMM",         */
/* bjdmk.com.cn, s3.2: element-wise operators -- activations, residual add  */
/* -- applied while the product is still on chip; "DeepGEMM: GPU high-      */
/* efficiency BLAS kernel library", s2.3: SwiGLU inside the MoE kernel).    */
/* Applied here in FP64 to the FP64 product:                                 */
/*   none: v;  relu: max(v, 0);  silu: v / (1 + e^-v);                        */
/*   gelu: v/2 (1 + erf(v / sqrt 2));                                         */
/*   swiglu: with B rows interleaved (row 2j gate, row 2j+1 up), output      */
/*     column j = silu(acc[2j]) * acc[2j+1], so the output has N/2 columns.  */
/* Then, if given, the BF16 residual [M][Nout] is added.                     */
/* ------------------------------------------------------------------------ */

static double silu(double v) { return v / (1.0 + exp(-v)); }

static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int orc_epilogue(const double *acc, int64_t M, int64_t N, int act, const uint16_t *residual,
                 double *out)
{
    int64_t m, j, n_out;
    if (!acc || !out || M < 0 || N < 0 || act < 0 || act > 4)
        return -1;
    if (act == 4 && N % 2 != 0)
        return -1;
    n_out = act == 4 ? N / 2 : N;
    for (m = 0; m < M; ++m)
        for (j = 0; j < n_out; ++j) {
            double v;
            if (act == 4) {
                v = silu(acc[m * N + 2 * j]) * acc[m * N + 2 * j + 1];
            } else {
                double a = acc[m * N + j];
                switch (act) {
                case 1: v = a > 0.0 ? a : 0.0; break;
                case 2: v = silu(a); break;
                case 3: v = 0.5 * a * (1.0 + erf(a / sqrt(2.0))); break;
                default: v = a; break;
                }
            }
            if (residual)
                v += bf16_value(residual[m * n_out + j]);
            out[m * n_out + j] = v;
        }
    return 0;
}
