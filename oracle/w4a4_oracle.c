/*
 * CPU oracle for the W4A4 MX projection GEMV.  TEST INFRASTRUCTURE ONLY:
 * nothing on the product path may link, load or call this file.  Only the
 * tests, the smoke check and the benchmark's CPU-baseline leg use it.
 *
 * The page "w4a4_proj/mx_plan.rs" plans an m-row W4A4 projection (m up to
 * 64, weights in 16-row tiles, K walked in 128-wide chunks) but states no
 * number format.  The reading used here is the OCP Microscaling (MX)
 * format its "mx" names point to, MXFP4:
 *   - elements are FP4 E2M1 (1 sign, 2 exponent bits with bias 1, 1
 *     mantissa bit; values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives;
 *     no infinities or NaNs), two per byte, the even element in the low
 *     nibble;
 *   - every 32 consecutive K elements of a row share one E8M0 scale byte:
 *     2^(e - 127), e = 255 being NaN (never generated).
 * Both the activations A [m, k] and the weight W [n, k] are MXFP4 with
 * their own scales, A scales [m, k/32] and W scales [n, k/32] row-major.
 *
 *   C[i][j] = RNE_bf16( sum_{b < K/32} sa[i][b] * sw[j][b] * sum_{t < 32} a[i][32b+t] * w[j][32b+t] )
 *
 * Everything is accumulated in IEEE double and rounded once to BF16
 * (round to nearest even) straight from double.  Each block's partial sum
 * is exact in double (products of E2M1 values have at most 3 significant
 * bits and |sum| <= 32 * 36); scaling by two powers of two is exact; only
 * the sum over blocks can round, and not at all for the moderate scales of
 * the tests.  Alongside C the oracle returns the double total and the bound
 * B = sum |a * w * sa * sw| that the parity tolerance is written in.
 *
 * Build: with w8a16_oracle.c into liboracle.so (gcc -O2, no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define W4A4_BLOCK 32u

uint16_t oracle_bf16_rne(double x);   /* w8a16_oracle.c */

/* FP4 E2M1 (4 low bits of `code`): sign s, exponent e (2 bits, bias 1),
 * mantissa m (1 bit).  e == 0 is subnormal: m * 0.5.  Otherwise
 * (1 + m/2) * 2^(e - 1). */
double oracle_e2m1_value(uint8_t code)
{
    unsigned s = (code >> 3) & 1u;
    unsigned e = (code >> 1) & 3u;
    unsigned m = code & 1u;
    double v = e == 0u ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -v : v;
}

/* E8M0 scale byte: 2^(e - 127); 0xFF is NaN. */
double oracle_e8m0_value(uint8_t e)
{
    if (e == 0xFFu)
        return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* Element t of a packed FP4 row: byte t/2, low nibble for even t. */
static double fp4_at(const uint8_t *row, uint32_t t)
{
    uint8_t byte = row[t >> 1];
    return oracle_e2m1_value((t & 1u) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15u));
}

/* One output: the block sums in ascending block order. */
static void w4a4_one(const uint8_t *arow, const uint8_t *asc, const uint8_t *wrow,
                     const uint8_t *wsc, uint32_t k, double *tot, double *bound)
{
    double t = 0.0, b = 0.0;
    for (uint32_t blk = 0; blk < k / W4A4_BLOCK; ++blk) {
        double p = 0.0, pb = 0.0;
        for (uint32_t u = 0; u < W4A4_BLOCK; ++u) {
            const uint32_t kk = blk * W4A4_BLOCK + u;
            const double prod = fp4_at(arow, kk) * fp4_at(wrow, kk);
            p += prod;
            pb += fabs(prod);
        }
        const double s = oracle_e8m0_value(asc[blk]) * oracle_e8m0_value(wsc[blk]);
        t += s * p;
        b += s * pb;
    }
    *tot = t;
    *bound = b;
}

/* Whole GEMM.  a: packed FP4, row i at byte offset i * a_row_stride / 2
 * (a_row_stride in elements, even); a_scale [m][k/32]; w: packed FP4
 * [n][k/2 bytes]; w_scale [n][k/32]; c: BF16 bits, row pitch c_row_stride
 * (only the first n of each row written); tot, bound: [m][n] (may be null).
 * Returns 0, or -1 for a shape it does not take. */
int oracle_w4a4_gemm(const uint8_t *a, uint32_t a_row_stride, const uint8_t *a_scale,
                     const uint8_t *w, const uint8_t *w_scale, uint16_t *c,
                     uint32_t c_row_stride, uint32_t m, uint32_t n, uint32_t k, double *tot,
                     double *bound, int nthreads)
{
    if (m == 0 || n == 0 || k == 0 || k % W4A4_BLOCK != 0 || a_row_stride < k ||
        a_row_stride % 2u != 0 || c_row_stride < n)
        return -1;
    const uint32_t kb = k / W4A4_BLOCK;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t idx = 0; idx < (int64_t)m * n; ++idx) {
        const uint32_t i = (uint32_t)(idx / n), j = (uint32_t)(idx % n);
        double t, b;
        w4a4_one(a + (size_t)i * (a_row_stride / 2u), a_scale + (size_t)i * kb,
                 w + (size_t)j * (k / 2u), w_scale + (size_t)j * kb, k, &t, &b);
        c[(size_t)i * c_row_stride + j] = oracle_bf16_rne(t);
        if (tot)
            tot[(size_t)i * n + j] = t;
        if (bound)
            bound[(size_t)i * n + j] = b;
    }
#ifndef _OPENMP
    (void)nthreads;
#endif
    return 0;
}

/* Selected outputs only, for shapes too large to compute whole: sample s is
 * C[rows[s]][cols[s]], operands as for oracle_w4a4_gemm.  c_out receives
 * BF16 bits, tot and bound doubles (each may be null).  Returns -1 for a
 * shape it does not take or an index out of range (before reading any
 * operand). */
int oracle_w4a4_gemm_at(const uint8_t *a, uint32_t a_row_stride, const uint8_t *a_scale,
                        const uint8_t *w, const uint8_t *w_scale, uint32_t m, uint32_t n,
                        uint32_t k, const uint32_t *rows, const uint32_t *cols, int64_t nsamp,
                        uint16_t *c_out, double *tot, double *bound, int nthreads)
{
    if (m == 0 || n == 0 || k == 0 || k % W4A4_BLOCK != 0 || a_row_stride < k ||
        a_row_stride % 2u != 0 || nsamp < 0)
        return -1;
    for (int64_t s = 0; s < nsamp; ++s)
        if (rows[s] >= m || cols[s] >= n)
            return -1;
    const uint32_t kb = k / W4A4_BLOCK;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t s = 0; s < nsamp; ++s) {
        const uint32_t i = rows[s], j = cols[s];
        double t, b;
        w4a4_one(a + (size_t)i * (a_row_stride / 2u), a_scale + (size_t)i * kb,
                 w + (size_t)j * (k / 2u), w_scale + (size_t)j * kb, k, &t, &b);
        if (c_out)
            c_out[s] = oracle_bf16_rne(t);
        if (tot)
            tot[s] = t;
        if (bound)
            bound[s] = b;
    }
#ifndef _OPENMP
    (void)nthreads;
#endif
    return 0;
}
