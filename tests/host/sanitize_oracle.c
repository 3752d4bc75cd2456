/* Host-only driver for the CPU oracle (oracle/w8a16_oracle.c and
 * oracle/w4a4_oracle.c), built with AddressSanitizer and
 * UndefinedBehaviorSanitizer (and without OpenMP) by the CPU test suite.
 * Every buffer is allocated to exactly the bytes its documented layout
 * covers -- the last row of a pitched operand only as long as the row --
 * so a read or write past the layout is reported.  Shapes: single rows,
 * ragged column counts, pitches longer than the row, several K blocks, the
 * sampled-output entry points, and the shapes each function rejects.
 * Every byte of every operand is random (NaN and Inf codes included), so
 * every decode path runs.  A sanitizer report aborts the run. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_e4m3_value(uint8_t code);
double oracle_bf16_value(uint16_t h);
uint16_t oracle_bf16_rne(double x);
uint8_t oracle_e4m3_rne(float x);
double oracle_e2m1_value(uint8_t code);
double oracle_e8m0_value(uint8_t e);
int oracle_w8a16_gemm(const uint16_t *a, uint32_t a_row_stride, const uint8_t *w,
                      const float *scale, uint16_t *c, uint32_t c_row_stride, uint32_t m,
                      uint32_t n, uint32_t k, double *tot, double *bound, int nthreads);
int oracle_w8a16_gemm_at(const uint16_t *a, uint32_t a_row_stride, const uint8_t *w,
                         const float *scale, uint32_t m, uint32_t n, uint32_t k,
                         const uint32_t *rows, const uint32_t *cols, int64_t nsamp,
                         uint16_t *c_out, double *tot, double *bound, int nthreads);
int oracle_act_quant(const uint16_t *a, uint32_t a_row_stride, uint32_t m, uint32_t k,
                     uint8_t *q, uint32_t q_row_stride, float *scales);
int oracle_w8a8_gemm(const uint8_t *qa, uint32_t qa_row_stride, const float *sa,
                     const uint8_t *w, const float *sw, uint16_t *c, uint32_t c_row_stride,
                     uint32_t m, uint32_t n, uint32_t k, double *tot, double *bound,
                     int nthreads);
int oracle_w8a8_gemm_at(const uint8_t *qa, uint32_t qa_row_stride, const float *sa,
                        const uint8_t *w, const float *sw, uint32_t m, uint32_t n, uint32_t k,
                        const uint32_t *rows, const uint32_t *cols, int64_t nsamp,
                        uint16_t *c_out, double *tot, double *bound, int nthreads);
int oracle_w4a4_gemm(const uint8_t *a, uint32_t a_row_stride, const uint8_t *a_scale,
                     const uint8_t *w, const uint8_t *w_scale, uint16_t *c,
                     uint32_t c_row_stride, uint32_t m, uint32_t n, uint32_t k, double *tot,
                     double *bound, int nthreads);
int oracle_w4a4_gemm_at(const uint8_t *a, uint32_t a_row_stride, const uint8_t *a_scale,
                        const uint8_t *w, const uint8_t *w_scale, uint32_t m, uint32_t n,
                        uint32_t k, const uint32_t *rows, const uint32_t *cols, int64_t nsamp,
                        uint16_t *c_out, double *tot, double *bound, int nthreads);

static uint64_t g_state = 0x13198a2e03707344ull;

/* xorshift64 (Marsaglia, "Xorshift RNGs", 2003) */
static uint32_t next_u32(void)
{
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return (uint32_t)(g_state >> 32);
}

static void *random_bytes(size_t bytes)
{
    uint8_t *p = malloc(bytes ? bytes : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    for (size_t i = 0; i < bytes; ++i)
        p[i] = (uint8_t)next_u32();
    return p;
}

/* Finite scales of either sign (the GEMMs' scale operands). */
static float *random_scales(size_t count)
{
    float *s = malloc(count ? count * sizeof(float) : 1);
    for (size_t i = 0; i < count; ++i)
        s[i] = ldexpf((float)(next_u32() % 1000 + 1) / 1000.0f, (int)(next_u32() % 16) - 8) *
               (next_u32() % 2 ? 1.0f : -1.0f);
    return s;
}

/* Finite BF16 activations (the quantizer's domain): random sign and
 * mantissa, exponent within +-20 of 1, zeros now and then. */
static uint16_t *random_bf16(size_t count)
{
    uint16_t *a = malloc(count ? count * 2 : 1);
    for (size_t i = 0; i < count; ++i) {
        const uint32_t r = next_u32();
        a[i] = r % 17 == 0 ? 0
                           : (uint16_t)(((r >> 31) << 15) | ((107 + (r >> 8) % 41) << 7) |
                                        (r & 0x7f));
    }
    return a;
}

static size_t pitched(uint32_t rows, uint32_t pitch, uint32_t row)
{
    return rows == 0 ? 0 : (size_t)(rows - 1) * pitch + row;
}

static int g_bad = 0;

static void expect_status(int got, int want, const char *what)
{
    if (got != want) {
        fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
        g_bad = 1;
    }
}

static void run_w8a16(uint32_t m, uint32_t n, uint32_t k, uint32_t pad_a, uint32_t pad_c)
{
    const uint32_t as = k + pad_a, cs = n + pad_c, nb = (n + 127) / 128, ks = k / 128;
    uint16_t *a = random_bytes(pitched(m, as, k) * 2);
    uint8_t *w = random_bytes((size_t)n * k);
    float *s = random_scales((size_t)nb * ks);
    uint16_t *c = malloc(pitched(m, cs, n) * 2);
    double *tot = malloc((size_t)m * n * sizeof(double));
    double *bnd = malloc((size_t)m * n * sizeof(double));
    expect_status(oracle_w8a16_gemm(a, as, w, s, c, cs, m, n, k, tot, bnd, 1), 0, "w8a16");
    uint32_t rows[3] = {0, m - 1, m / 2}, cols[3] = {n - 1, 0, n / 2};
    uint16_t co[3];
    double t3[3], b3[3];
    expect_status(oracle_w8a16_gemm_at(a, as, w, s, m, n, k, rows, cols, 3, co, t3, b3, 1), 0,
                  "w8a16 sampled");
    rows[2] = m;  /* out of range: rejected before any read */
    expect_status(oracle_w8a16_gemm_at(a, as, w, s, m, n, k, rows, cols, 3, co, t3, b3, 1), -1,
                  "w8a16 sampled, row out of range");

    /* quantize the same activations and run the W8A8 GEMM on them */
    const uint32_t qs = k + 16 * (pad_a % 3);
    uint16_t *af = random_bf16(pitched(m, as, k));
    uint8_t *q = malloc(pitched(m, qs, k));
    float *sa = malloc((size_t)m * ks * sizeof(float));
    expect_status(oracle_act_quant(af, as, m, k, q, qs, sa), 0, "act quant");
    expect_status(oracle_w8a8_gemm(q, qs, sa, w, s, c, cs, m, n, k, tot, bnd, 1), 0, "w8a8");
    rows[2] = m / 2;
    expect_status(oracle_w8a8_gemm_at(q, qs, sa, w, s, m, n, k, rows, cols, 3, co, t3, b3, 1),
                  0, "w8a8 sampled");
    free(af);
    free(q);
    free(sa);
    free(a);
    free(w);
    free(s);
    free(c);
    free(tot);
    free(bnd);
}

static void run_w4a4(uint32_t m, uint32_t n, uint32_t k, uint32_t pad_a, uint32_t pad_c)
{
    const uint32_t as = k + 2 * pad_a, cs = n + pad_c, g = k / 32;
    uint8_t *a = random_bytes(pitched(m, as / 2, k / 2));
    uint8_t *sa = random_bytes((size_t)m * g);
    uint8_t *w = random_bytes((size_t)n * k / 2);
    uint8_t *sw = random_bytes((size_t)n * g);
    uint16_t *c = malloc(pitched(m, cs, n) * 2);
    double *tot = malloc((size_t)m * n * sizeof(double));
    double *bnd = malloc((size_t)m * n * sizeof(double));
    expect_status(oracle_w4a4_gemm(a, as, sa, w, sw, c, cs, m, n, k, tot, bnd, 1), 0, "w4a4");
    expect_status(oracle_w4a4_gemm(a, as, sa, w, sw, c, cs, m, n, k, NULL, NULL, 1), 0,
                  "w4a4 without diagnostics");
    uint32_t rows[3] = {m - 1, 0, m / 2}, cols[3] = {0, n - 1, n / 2};
    uint16_t co[3];
    double t3[3], b3[3];
    expect_status(oracle_w4a4_gemm_at(a, as, sa, w, sw, m, n, k, rows, cols, 3, co, t3, b3, 1),
                  0, "w4a4 sampled");
    cols[1] = n;  /* out of range: rejected before any read */
    expect_status(oracle_w4a4_gemm_at(a, as, sa, w, sw, m, n, k, rows, cols, 3, co, t3, b3, 1),
                  -1, "w4a4 sampled, column out of range");
    free(a);
    free(sa);
    free(w);
    free(sw);
    free(c);
    free(tot);
    free(bnd);
}

int main(void)
{
    for (uint32_t x = 0; x < 256; ++x) {
        volatile double v = oracle_e4m3_value((uint8_t)x) + oracle_e2m1_value((uint8_t)(x & 15)) +
                            oracle_e8m0_value((uint8_t)x);
        (void)v;
    }
    for (uint32_t h = 0; h < 65536; ++h) {
        const double v = oracle_bf16_value((uint16_t)h);
        volatile uint16_t r = oracle_bf16_rne(v);
        volatile uint8_t e = oracle_e4m3_rne((float)v);
        (void)r;
        (void)e;
    }

    static const uint32_t shapes[][5] = {
        /* m, n, k, A pitch padding, C pitch padding */
        {1, 1, 128, 0, 0},    {1, 17, 256, 8, 3},    {3, 129, 128, 0, 1},
        {5, 130, 384, 24, 0}, {16, 16, 128, 8, 16},  {17, 255, 256, 0, 0},
        {33, 64, 512, 40, 7}, {2, 300, 1024, 8, 0},
    };
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) {
        run_w8a16(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3], shapes[i][4]);
        run_w4a4(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3], shapes[i][4]);
        run_w4a4(shapes[i][0], shapes[i][1], 32 * (1 + i), shapes[i][3], shapes[i][4]);
    }

    /* rejected shapes: nothing is read or written */
    uint16_t c1;
    expect_status(oracle_w8a16_gemm(NULL, 128, NULL, NULL, &c1, 1, 0, 1, 128, NULL, NULL, 1), -1,
                  "w8a16 m=0");
    expect_status(oracle_w8a16_gemm(NULL, 100, NULL, NULL, &c1, 1, 1, 1, 100, NULL, NULL, 1), -1,
                  "w8a16 k=100");
    expect_status(oracle_w8a16_gemm(NULL, 64, NULL, NULL, &c1, 1, 1, 1, 128, NULL, NULL, 1), -1,
                  "w8a16 short A pitch");
    expect_status(oracle_act_quant(NULL, 128, 1, 128, NULL, 64, NULL), -1, "quant short pitch");
    expect_status(oracle_w4a4_gemm(NULL, 33, NULL, NULL, NULL, &c1, 1, 1, 1, 32, NULL, NULL, 1),
                  -1, "w4a4 odd pitch");
    expect_status(oracle_w4a4_gemm(NULL, 48, NULL, NULL, NULL, &c1, 1, 1, 1, 48, NULL, NULL, 1),
                  -1, "w4a4 k=48");

    printf("oracle sweep done, %s\n", g_bad ? "STATUS MISMATCH" : "ok");
    return g_bad;
}
