/*
 * CPU oracle for the block-scaled FP8 W8A16 GEMM.  TEST INFRASTRUCTURE ONLY:
 * nothing on the product path may link, load or call this file.  Only the
 * tests, the smoke check and the benchmark's CPU-baseline leg use it.
 *
 * What it computes (page "w8a16_gemm_pipelined_m32.rs", the doc comment of
 * `w8a16_gemm_pipelined_m32_strided` and of `W8A16_M32_K_BLOCK`, and the
 * module doc's "Numerics" paragraph):
 *
 *   C[i][j] = RNE_bf16( sum_{b < K/128} S[j/128][b] * sum_{t < 128} A[i][128b+t] * W[j][128b+t] )
 *
 *   A  BF16  [M, a_row_stride]   only the first K elements of each row are read
 *   W  E4M3  [N, K]              row-major, contiguous
 *   S  FP32  [ceil(N/128), K/128] row-major, one scale per 128x128 weight block
 *   C  BF16  [M, c_row_stride]   only the first N elements of each row are written
 *
 * The scale of a block is applied once to that block's 128-wide partial dot
 * product (the fold point of one FP8 scale block per K step), never to
 * single weights.  Everything is accumulated in IEEE double and rounded once,
 * directly from double, to BF16 with round-to-nearest-even.
 *
 * Readings of points the page leaves open:
 *   - "FP8 E4M3" is the OCP E4M3FN encoding (bias 7, largest finite 448,
 *     S.1111.111 is NaN, no infinities, subnormals f * 2^-9).
 *   - The scale tensor is row-major with ceil(N/128) rows, so a ragged last
 *     N block still has a scale row.
 *   - NaN codes are outside the contract; the oracle propagates them as NaN.
 *
 * Each product A*W is exact in double (8-bit x 4-bit significands), so the
 * only roundings are the double sums, the double product scale*partial and
 * the final BF16 rounding.  Alongside C the oracle can return the double
 * total before rounding and the bound B[i][j] = sum |A*W| * |S| that the
 * parity tolerance is written in.
 *
 * The second part of the file (after the W8A16 GEMM) is the FP8 activation
 * quantizer and the W8A8 GEMM; its readings are stated there.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_K_BLOCK 128u

/* OCP E4M3FN decode of one byte: sign s, exponent e (4 bits, bias 7),
 * fraction f (3 bits).  e == 0 is subnormal: f * 2^-9.  e == 15 with f == 7
 * is NaN.  Otherwise (1 + f/8) * 2^(e-7) == (8 + f) * 2^(e-10). */
double oracle_e4m3_value(uint8_t code)
{
    unsigned s = code >> 7;
    unsigned e = (code >> 3) & 15u;
    unsigned f = code & 7u;
    double v;
    if (e == 15u && f == 7u)
        return NAN;
    if (e == 0u)
        v = ldexp((double)f, -9);
    else
        v = ldexp((double)(8u + f), (int)e - 10);
    return s ? -v : v;
}

/* BF16 is the top half of an IEEE binary32: widen the bits and read it. */
double oracle_bf16_value(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Round a double to the nearest BF16, ties to even, in one step (never via
 * float, which would round twice).  BF16 keeps 8 significant bits; its
 * exponent range is binary32's, so below 2^-126 the spacing is fixed at
 * 2^-133.  Results above the largest finite BF16 become infinity. */
uint16_t oracle_bf16_rne(double x)
{
    uint32_t bits;
    float f;
    double a, q, r, v;
    int ex, e;

    if (isnan(x))
        return 0x7FC0u;
    if (x == 0.0)
        return signbit(x) ? 0x8000u : 0x0000u;
    if (isinf(x))
        return signbit(x) ? 0xFF80u : 0x7F80u;

    a = fabs(x);
    frexp(a, &ex);          /* a = m * 2^ex, m in [0.5, 1) */
    e = ex - 1;             /* floor(log2 a) */
    if (e < -126)
        e = -126;
    q = ldexp(1.0, e - 7);  /* spacing of BF16 values in a's binade */
    r = nearbyint(a / q);   /* a/q is exact; default mode rounds ties to even */
    v = r * q;              /* exact: r < 2^9 */
    if (v > ldexp(255.0, 120))   /* largest finite BF16: (2 - 2^-7) * 2^127 */
        return signbit(x) ? 0xFF80u : 0x7F80u;
    f = (float)v;           /* exact: v is a BF16 value */
    memcpy(&bits, &f, sizeof bits);
    bits >>= 16;
    if (signbit(x))
        bits |= 0x8000u;
    return (uint16_t)bits;
}

/* The 256-entry decode table is just oracle_e4m3_value() evaluated once per
 * code, so the inner loop does not re-derive the same 256 values. */
static void oracle_e4m3_table(double table[256])
{
    for (unsigned c = 0; c < 256u; ++c)
        table[c] = oracle_e4m3_value((uint8_t)c);
}

/* One output element: blocks in ascending order, elements in ascending order
 * inside each block, the block's scale applied once to its partial sum. */
static void oracle_element(const uint16_t *a, uint32_t a_row_stride,
                           const uint8_t *w, const float *scale,
                           uint32_t i, uint32_t j, uint32_t k,
                           const double table[256],
                           double *tot_out, double *bound_out)
{
    const uint32_t kb = k / ORACLE_K_BLOCK;
    const uint16_t *arow = a + (size_t)i * a_row_stride;
    const uint8_t *wrow = w + (size_t)j * k;
    const float *srow = scale + (size_t)(j / ORACLE_K_BLOCK) * kb;
    double tot = 0.0, bound = 0.0;

    for (uint32_t b = 0; b < kb; ++b) {
        double p = 0.0, pabs = 0.0;
        for (uint32_t t = 0; t < ORACLE_K_BLOCK; ++t) {
            uint32_t kk = b * ORACLE_K_BLOCK + t;
            double prod = oracle_bf16_value(arow[kk]) * table[wrow[kk]];
            p += prod;
            pabs += fabs(prod);
        }
        double s = (double)srow[b];
        tot += s * p;
        bound += fabs(s) * pabs;
    }
    *tot_out = tot;
    if (bound_out)
        *bound_out = bound;
}

/* Full GEMM.  c (if non-null) receives BF16 bits at c_row_stride; tot and
 * bound (if non-null) receive dense [m, n] doubles.  Returns 0, or -1 when
 * the shape is outside the operation's domain (m or n zero, k not a positive
 * multiple of 128, a pitch shorter than the row it must hold). */
int oracle_w8a16_gemm(const uint16_t *a, uint32_t a_row_stride,
                      const uint8_t *w, const float *scale,
                      uint16_t *c, uint32_t c_row_stride,
                      uint32_t m, uint32_t n, uint32_t k,
                      double *tot, double *bound, int nthreads)
{
    double table[256];
    int64_t total, idx;

    if (m == 0 || n == 0 || k == 0 || k % ORACLE_K_BLOCK != 0 ||
        a_row_stride < k || (c && c_row_stride < n))
        return -1;
    oracle_e4m3_table(table);
    total = (int64_t)m * n;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (idx = 0; idx < total; ++idx) {
        uint32_t i = (uint32_t)(idx / n), j = (uint32_t)(idx % n);
        double t, bnd;
        oracle_element(a, a_row_stride, w, scale, i, j, k, table, &t, &bnd);
        if (c)
            c[(size_t)i * c_row_stride + j] = oracle_bf16_rne(t);
        if (tot)
            tot[idx] = t;
        if (bound)
            bound[idx] = bnd;
    }
    (void)nthreads;
    return 0;
}

/* Selected outputs only, for shapes too large to compute whole: sample s is
 * C[rows[s]][cols[s]].  c_out receives BF16 bits, tot/bound doubles (each
 * may be null).  Returns -1 for an invalid shape or an index out of range. */
int oracle_w8a16_gemm_at(const uint16_t *a, uint32_t a_row_stride,
                         const uint8_t *w, const float *scale,
                         uint32_t m, uint32_t n, uint32_t k,
                         const uint32_t *rows, const uint32_t *cols,
                         int64_t nsamp, uint16_t *c_out,
                         double *tot, double *bound, int nthreads)
{
    double table[256];
    int64_t s;
    int bad = 0;

    if (m == 0 || n == 0 || k == 0 || k % ORACLE_K_BLOCK != 0 ||
        a_row_stride < k)
        return -1;
    for (s = 0; s < nsamp; ++s)
        if (rows[s] >= m || cols[s] >= n)
            bad = 1;
    if (bad)
        return -1;
    oracle_e4m3_table(table);
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (s = 0; s < nsamp; ++s) {
        double t, bnd;
        oracle_element(a, a_row_stride, w, scale, rows[s], cols[s], k,
                       table, &t, &bnd);
        if (c_out)
            c_out[s] = oracle_bf16_rne(t);
        if (tot)
            tot[s] = t;
        if (bound)
            bound[s] = bnd;
    }
    (void)nthreads;
    return 0;
}

/* Threads the OpenMP runtime would use for a parallel region. */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------
 * FP8 activation quantizer and W8A8 GEMM (page "fp8_act_quant.rs": one
 * quantization group is 128 K elements of one token; the page gives the
 * grouping, not the arithmetic).  Reading taken for the arithmetic, the
 * same rule as the weight blocks' scales: per (token, group)
 *     s = amax / 448            (binary32 division, 448 = largest E4M3FN)
 *     code_t = E4M3_RNE(clamp(x_t / s, -448, 448))   (binary32 division)
 * and an all-zero group gets s = 0 and +0 codes.  Both divisions are single
 * precision because the codes are integers decided by them: the kernel and
 * the oracle must take that decision in the same precision.
 * ------------------------------------------------------------------------ */

/* OCP E4M3FN code nearest to x, ties to even, saturating to +-448 (NaN ->
 * 0x7F).  Zero keeps its sign (-0 -> 0x80), and so does a value that rounds
 * to zero.  Below 2^-6 the spacing is the subnormal 2^-9; in binade
 * [2^e, 2^(e+1)) it is 2^(e-3).  a / spacing is exact in double. */
uint8_t oracle_e4m3_rne(float x)
{
    double a, r;
    int ex, e;
    unsigned code;
    const unsigned sign = signbit(x) ? 0x80u : 0u;

    if (isnan(x))
        return 0x7Fu;
    a = fabs((double)x);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7Eu);
    if (a < ldexp(1.0, -6)) {
        r = nearbyint(a / ldexp(1.0, -9));      /* 0..8; 8 is the code of 2^-6 */
        return (uint8_t)(sign | (unsigned)r);
    }
    frexp(a, &ex);
    e = ex - 1;                                 /* floor(log2 a), -6..8 */
    r = nearbyint(a / ldexp(1.0, e - 3));       /* 8..16 */
    if (r == 16.0) {
        r = 8.0;
        e += 1;
    }
    code = ((unsigned)(e + 7) << 3) | ((unsigned)r - 8u);
    if (code > 0x7Eu)
        code = 0x7Eu;
    return (uint8_t)(sign | code);
}

/* Quantize A (BF16 [m, a_row_stride], first k of each row) to codes
 * q [m, q_row_stride] and scales [m, k/128] (row-major). */
int oracle_act_quant(const uint16_t *a, uint32_t a_row_stride, uint32_t m, uint32_t k,
                     uint8_t *q, uint32_t q_row_stride, float *scales)
{
    const uint32_t groups = k / ORACLE_K_BLOCK;

    if (m == 0 || k == 0 || k % ORACLE_K_BLOCK != 0 || a_row_stride < k ||
        q_row_stride < k)
        return -1;
    for (uint32_t i = 0; i < m; ++i) {
        for (uint32_t g = 0; g < groups; ++g) {
            const uint16_t *x = a + (size_t)i * a_row_stride + (size_t)g * ORACLE_K_BLOCK;
            uint8_t *out = q + (size_t)i * q_row_stride + (size_t)g * ORACLE_K_BLOCK;
            float amax = 0.0f, s;
            for (uint32_t t = 0; t < ORACLE_K_BLOCK; ++t) {
                float v = (float)oracle_bf16_value(x[t]);   /* exact */
                if (fabsf(v) > amax)
                    amax = fabsf(v);
            }
            s = amax / 448.0f;
            scales[(size_t)i * groups + g] = s;
            for (uint32_t t = 0; t < ORACLE_K_BLOCK; ++t) {
                float y;
                if (s == 0.0f) {
                    out[t] = 0u;
                    continue;
                }
                y = (float)oracle_bf16_value(x[t]) / s;
                if (y > 448.0f)
                    y = 448.0f;
                if (y < -448.0f)
                    y = -448.0f;
                out[t] = oracle_e4m3_rne(y);
            }
        }
    }
    return 0;
}

/* One W8A8 output: blocks in ascending order, each block's exact partial
 * dot product of decoded codes times the product of its two scales (A's for
 * the row and K step, W's for the 128x128 weight block), in double. */
static void oracle_w8a8_element(const uint8_t *qa, uint32_t qa_row_stride,
                                const float *sa, const uint8_t *w, const float *sw,
                                uint32_t i, uint32_t j, uint32_t k,
                                const double table[256], double *tot_out,
                                double *bound_out)
{
    const uint32_t kb = k / ORACLE_K_BLOCK;
    const uint8_t *arow = qa + (size_t)i * qa_row_stride;
    const uint8_t *wrow = w + (size_t)j * k;
    const float *swrow = sw + (size_t)(j / ORACLE_K_BLOCK) * kb;
    const float *sarow = sa + (size_t)i * kb;
    double tot = 0.0, bound = 0.0;

    for (uint32_t b = 0; b < kb; ++b) {
        double p = 0.0, pabs = 0.0;
        for (uint32_t t = 0; t < ORACLE_K_BLOCK; ++t) {
            uint32_t kk = b * ORACLE_K_BLOCK + t;
            double prod = table[arow[kk]] * table[wrow[kk]];
            p += prod;
            pabs += fabs(prod);
        }
        double s = (double)sarow[b] * (double)swrow[b];
        tot += s * p;
        bound += fabs(s) * pabs;
    }
    *tot_out = tot;
    if (bound_out)
        *bound_out = bound;
}

/* Full W8A8 GEMM: qa E4M3 [m, qa_row_stride], sa FP32 [m, k/128], w E4M3
 * [n, k], sw FP32 [ceil(n/128), k/128]; outputs as oracle_w8a16_gemm. */
int oracle_w8a8_gemm(const uint8_t *qa, uint32_t qa_row_stride, const float *sa,
                     const uint8_t *w, const float *sw, uint16_t *c, uint32_t c_row_stride,
                     uint32_t m, uint32_t n, uint32_t k, double *tot, double *bound,
                     int nthreads)
{
    double table[256];
    int64_t total, idx;

    if (m == 0 || n == 0 || k == 0 || k % ORACLE_K_BLOCK != 0 ||
        qa_row_stride < k || (c && c_row_stride < n))
        return -1;
    oracle_e4m3_table(table);
    total = (int64_t)m * n;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (idx = 0; idx < total; ++idx) {
        uint32_t i = (uint32_t)(idx / n), j = (uint32_t)(idx % n);
        double t, bnd;
        oracle_w8a8_element(qa, qa_row_stride, sa, w, sw, i, j, k, table, &t, &bnd);
        if (c)
            c[(size_t)i * c_row_stride + j] = oracle_bf16_rne(t);
        if (tot)
            tot[idx] = t;
        if (bound)
            bound[idx] = bnd;
    }
    (void)nthreads;
    return 0;
}

/* Selected W8A8 outputs C[rows[s]][cols[s]]. */
int oracle_w8a8_gemm_at(const uint8_t *qa, uint32_t qa_row_stride, const float *sa,
                        const uint8_t *w, const float *sw, uint32_t m, uint32_t n,
                        uint32_t k, const uint32_t *rows, const uint32_t *cols,
                        int64_t nsamp, uint16_t *c_out, double *tot, double *bound,
                        int nthreads)
{
    double table[256];
    int64_t s;

    if (m == 0 || n == 0 || k == 0 || k % ORACLE_K_BLOCK != 0 || qa_row_stride < k)
        return -1;
    for (s = 0; s < nsamp; ++s)
        if (rows[s] >= m || cols[s] >= n)
            return -1;
    oracle_e4m3_table(table);
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (s = 0; s < nsamp; ++s) {
        double t, bnd;
        oracle_w8a8_element(qa, qa_row_stride, sa, w, sw, rows[s], cols[s], k, table, &t,
                            &bnd);
        if (c_out)
            c_out[s] = oracle_bf16_rne(t);
        if (tot)
            tot[s] = t;
        if (bound)
            bound[s] = bnd;
    }
    (void)nthreads;
    return 0;
}
