/*
 * Host sanitizer driver for the oracle and the input generators: every
 * exported function on small, ragged and empty shapes, both input types,
 * rotation on and off, with each buffer allocated to its exact size, so that
 * AddressSanitizer sees any access past it and UndefinedBehaviorSanitizer any
 * overflow, bad shift or invalid conversion; then slices of the CPU sweeps and
 * division proofs (tests/helpers/sweeps.c, fastdiv.c).  A few anchors of the
 * format are checked along the way (the pins themselves live in
 * test_oracle_pins.py).
 * Test code: built with -fsanitize=address,undefined and run by
 * tests/test_sanitizers_cpu.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* oracle/nvfp4_oracle.c */
void oracle_rotate16(const float *x, float *y);
uint8_t oracle_e2m1_code(float v);
float oracle_e4m3_value(uint8_t b);
uint8_t oracle_e4m3_byte(float v);
float oracle_global_scale(float amax);
float oracle_amax(const void *x, int is_f32, int64_t rows, int64_t cols, int rotate, int nthreads);
int oracle_quantize(const void *x, int is_f32, int64_t rows, int64_t cols, int rotate, uint8_t *q, uint8_t *s,
                    float *g_out, float *amax_out, int nthreads);
int oracle_quantize_given_scale(const void *x, int is_f32, int64_t rows, int64_t cols, int rotate, float g,
                                uint8_t *q, uint8_t *s, int nthreads);
void oracle_dequant_f64(const uint8_t *q, const uint8_t *s, float g, int64_t rows, int64_t cols, int rotate,
                        double *out, int nthreads);
double oracle_roundtrip_error(const void *x, int is_f32, int64_t rows, int64_t cols, int rotate,
                              const uint8_t *q, const uint8_t *s, float g, const uint8_t *col_mask,
                              int nthreads);
void oracle_e2m1_code_array(const float *v, int64_t n, uint8_t *out, int nthreads);
void oracle_e4m3_byte_array(const float *v, int64_t n, uint8_t *out, int nthreads);
void oracle_e2m1_code_bits(uint32_t lo, uint32_t hi, uint8_t *out, int nthreads);
void oracle_e4m3_byte_bits(uint32_t lo, uint32_t hi, uint8_t *out, int nthreads);
uint8_t oracle_e8m0_byte(float t);
float oracle_e8m0_value(uint8_t b);
int oracle_mx_quantize(const void *x, int is_f32, int64_t rows, int64_t cols, int rotate, uint8_t *q, uint8_t *s,
                       int nthreads);
void oracle_mx_dequant_f64(const uint8_t *q, const uint8_t *s, int64_t rows, int64_t cols, int rotate,
                           double *out, int nthreads);
double oracle_mx_roundtrip_error(const void *x, int is_f32, int64_t rows, int64_t cols, int rotate,
                                 const uint8_t *q, const uint8_t *s, int nthreads);
int oracle_rotate_tensor(const void *x, int is_f32, int64_t rows, int64_t cols, float *y, int nthreads);
int oracle_rotate_matrix(const void *x, int is_f32, int64_t rows, int64_t cols, const float *r, float *y,
                         int nthreads);
int64_t oracle_swizzled_scale_bytes(int64_t rows, int64_t cb);
void oracle_swizzle_scales(const uint8_t *s, int64_t rows, int64_t cb, uint8_t *out);

/* synth/synth.c */
void synth_normal_f64(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, double *out);
void synth_uniform_f64(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, double *out);
void synth_round_bf16(const double *in, int64_t n, uint16_t *out);
void synth_normal_bf16(uint64_t seed, uint64_t stream, int64_t n, double scale, uint16_t *out);
void synth_normal_f32(uint64_t seed, uint64_t stream, int64_t n, double scale, float *out);
int synth_gauss_outliers(uint64_t seed, int64_t rows, int64_t cols, int64_t n_out, double lo, double hi,
                         uint16_t *out, int64_t *picked_out);
int synth_t3_lognormal(uint64_t seed, int64_t rows, int64_t cols, uint16_t *out);
int synth_silu_ties(uint64_t seed, int64_t rows, int64_t cols, int rotate, uint16_t *out, int64_t *anchor_block,
                    int64_t *n_tie, uint8_t *tie_flags);
int synth_kv_heads(uint64_t seed, int64_t tokens, int64_t heads, int64_t dim, float *out, uint8_t *block_kind);

/* tests/helpers/sweeps.c and tests/helpers/fastdiv.c, on small ranges */
long long sweep_e4m3_range(uint32_t lo, uint32_t hi, uint32_t *first);
long long sweep_e4m3_linear(uint32_t lo, uint32_t hi, uint32_t stride, uint32_t *first);
long long verify_div_const(float c, uint32_t lo, uint32_t hi, uint32_t *ex);
long long verify_random_codes2(int64_t n, uint64_t seed);
long long verify_recip_tail(int lo_exp, int hi_exp, uint32_t *ex_d);
long long verify_global_scale(uint32_t lo, uint32_t hi, uint32_t *ex);

static int failures = 0;
#define CHECK(c, ...)                                      \
    do {                                                   \
        if (!(c)) {                                        \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                  \
            fprintf(stderr, "\n");                         \
            failures++;                                    \
        }                                                  \
    } while (0)

/* malloc of exactly n bytes (n may be 0: one byte, never touched) */
static void *xmalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

/* The whole oracle on one tensor; returns nothing, checks invariants. */
static void run_tensor(const void *x, int is_f32, int64_t rows, int64_t cols)
{
    const int64_t n = rows * cols, nb = n / 16;
    for (int rotate = 0; rotate < 2; rotate++) {
        uint8_t *q = xmalloc((size_t)(n / 2)), *s = xmalloc((size_t)nb);
        uint8_t *q4 = xmalloc((size_t)(n / 2)), *s4 = xmalloc((size_t)nb);
        float g = 0, a = 0, g4 = 0, a4 = 0;
        CHECK(oracle_quantize(x, is_f32, rows, cols, rotate, q, s, &g, &a, 1) == 0, "quantize");
        CHECK(oracle_quantize(x, is_f32, rows, cols, rotate, q4, s4, &g4, &a4, 4) == 0, "quantize 4 threads");
        CHECK(memcmp(q, q4, (size_t)(n / 2)) == 0 && memcmp(s, s4, (size_t)nb) == 0 && g == g4 && a == a4,
              "thread-count invariance %lldx%lld", (long long)rows, (long long)cols);
        CHECK(g > 0.0f, "global scale positive");
        for (int64_t b = 0; b < nb; b++)
            CHECK(s[b] <= 0x7E, "scale byte %d", s[b]);
        CHECK(oracle_amax(x, is_f32, rows, cols, rotate, 2) == a, "amax alone");
        CHECK(oracle_quantize_given_scale(x, is_f32, rows, cols, rotate, g, q4, s4, 3) == 0, "given scale");
        CHECK(memcmp(q, q4, (size_t)(n / 2)) == 0 && memcmp(s, s4, (size_t)nb) == 0, "given scale bytes");
        CHECK(oracle_quantize_given_scale(x, is_f32, rows, cols, rotate, g * 1e-6f, q4, s4, 2) == 0,
              "given small scale");
        double *y = xmalloc((size_t)n * sizeof(double));
        oracle_dequant_f64(q, s, g, rows, cols, rotate, y, 2);
        double e = oracle_roundtrip_error(x, is_f32, rows, cols, rotate, q, s, g, NULL, 2);
        CHECK(!(e < 0.0), "round-trip error %g", e);
        uint8_t *mask = xmalloc((size_t)cols);
        for (int64_t c = 0; c < cols; c++)
            mask[c] = (uint8_t)(c % 3 != 0);
        e = oracle_roundtrip_error(x, is_f32, rows, cols, rotate, q, s, g, mask, 2);
        CHECK(!(e < 0.0), "masked round-trip error %g", e);
        free(mask);
        free(y);
        if (cols % 32 == 0) {
            uint8_t *ms = xmalloc((size_t)(n / 32));
            CHECK(oracle_mx_quantize(x, is_f32, rows, cols, rotate, q4, ms, 2) == 0, "mx quantize");
            double *ym = xmalloc((size_t)n * sizeof(double));
            oracle_mx_dequant_f64(q4, ms, rows, cols, rotate, ym, 2);
            (void)oracle_mx_roundtrip_error(x, is_f32, rows, cols, rotate, q4, ms, 2);
            free(ym);
            free(ms);
        }
        const int64_t sw = oracle_swizzled_scale_bytes(rows, cols / 16);
        uint8_t *ss = xmalloc((size_t)sw);
        oracle_swizzle_scales(s, rows, cols / 16, ss);
        free(ss);
        free(q);
        free(s);
        free(q4);
        free(s4);
    }
    float *yr = xmalloc((size_t)n * sizeof(float)), *ym = xmalloc((size_t)n * sizeof(float));
    float r[256];
    for (int i = 0; i < 256; i++)
        r[i] = (i / 16 == i % 16) ? 1.0f : 0.0f;
    CHECK(oracle_rotate_tensor(x, is_f32, rows, cols, yr, 2) == 0, "rotate tensor");
    CHECK(oracle_rotate_matrix(x, is_f32, rows, cols, r, ym, 2) == 0, "rotate matrix");
    for (int64_t i = 0; i < n; i++) {
        float v;
        if (is_f32) {
            v = ((const float *)x)[i];
        } else {
            uint32_t u = (uint32_t)((const uint16_t *)x)[i] << 16;
            memcpy(&v, &u, 4);
        }
        CHECK(memcmp(&ym[i], &v, 4) == 0 || (ym[i] == 0.0f && v == 0.0f), "identity rotation at %lld",
              (long long)i);
    }
    free(yr);
    free(ym);
}

int main(void)
{
    /* format anchors */
    static const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
    static const uint8_t want[7] = {0, 2, 2, 4, 4, 6, 6};
    for (int k = 0; k < 7; k++)
        CHECK(oracle_e2m1_code(mids[k]) == want[k], "E2M1 midpoint %g", mids[k]);
    CHECK(oracle_e2m1_code(-0.0f) == 0 && oracle_e2m1_code(-1e-30f) == 8, "E2M1 sign rule");
    CHECK(oracle_e4m3_byte(448.0f) == 0x7E && oracle_e4m3_byte(1e30f) == 0x7E, "E4M3 448");
    CHECK(oracle_e4m3_value(0x08) == 0x1p-6f && oracle_e4m3_value(0x01) == 0x1p-9f, "E4M3 anchors");
    CHECK(oracle_global_scale(0.0f) == 1.0f, "zero amax");
    CHECK(oracle_e8m0_value(oracle_e8m0_byte(1.0f)) == 1.0f, "E8M0 of 1");
    float e16[16], h16[16];
    for (int i = 0; i < 16; i++)
        e16[i] = (float)(i == 3);
    oracle_rotate16(e16, h16);
    for (int i = 0; i < 16; i++)
        CHECK(fabsf(h16[i]) == 0.25f, "H16 column entry %d", i);

    /* element arrays and bit ranges */
    float v[1000];
    uint8_t o[1000];
    for (int i = 0; i < 1000; i++)
        v[i] = (float)(i - 500) * 0.0137f;
    oracle_e2m1_code_array(v, 1000, o, 3);
    oracle_e4m3_byte_array(v + 500, 500, o, 3);
    oracle_e2m1_code_bits(0x3E800000u, 0x3E8003E7u, o, 2);
    oracle_e4m3_byte_bits(0x43DF0000u, 0x43DF03E7u, o, 2);

    /* the CPU proof helpers, on slices of their full ranges */
    uint32_t first = 0;
    CHECK(sweep_e4m3_range(0x3B000000u, 0x3B03FFFFu, &first) == 0, "E4M3 sweep slice");
    CHECK(sweep_e4m3_linear(0, 0x44800000u, 104729, &first) == 0, "E4M3 strided slice");
    CHECK(verify_div_const(6.0f, 0x40000000u, 0x4003FFFFu, &first) == 0, "divide by 6 slice");
    CHECK(verify_div_const(24.0f, 0x40000000u, 0x4003FFFFu, &first) == 0, "divide by 24 slice");
    CHECK(verify_random_codes2(200000, 7) == 0, "two-word quotient sample");
    CHECK(verify_recip_tail(0, 1, &first) == 0, "corrected reciprocal tail, one binade");
    CHECK(verify_global_scale(0x3F800000u, 0x3F83FFFFu, &first) == 0, "global scale slice");

    /* generators and the oracle on their tensors */
    const int64_t shapes[][2] = {{1, 16}, {3, 48}, {5, 1024}, {17, 1040}, {2, 4096}, {0, 64}, {7, 32}};
    for (size_t t = 0; t < sizeof shapes / sizeof shapes[0]; t++) {
        const int64_t rows = shapes[t][0], cols = shapes[t][1], n = rows * cols;
        uint16_t *xb = xmalloc((size_t)n * 2);
        float *xf = xmalloc((size_t)n * 4);
        double *d = xmalloc((size_t)n * sizeof(double));
        synth_normal_f64(1, 2, 3, n, d);
        synth_uniform_f64(1, 3, 0, n, d);
        synth_round_bf16(d, n, xb);
        synth_normal_bf16(4, 5, n, 2.0, xb);
        synth_normal_f32(4, 6, n, 3.0, xf);
        run_tensor(xb, 0, rows, cols);
        run_tensor(xf, 1, rows, cols);
        if (n > 0) {
            int64_t picked[4];
            CHECK(synth_gauss_outliers(0, rows, cols, cols < 4 ? cols : 4, 50.0, 50.0, xb, picked) == 0, "outliers");
            run_tensor(xb, 0, rows, cols);
            CHECK(synth_t3_lognormal(0, rows, cols, xb) == 0, "t3");
            run_tensor(xb, 0, rows, cols);
            int64_t anchor = -1, nt = -1;
            uint8_t *flags = xmalloc((size_t)(n / 16));
            for (int rot = 0; rot < 2; rot++) {
                CHECK(synth_silu_ties(0, rows, cols, rot, xb, &anchor, &nt, flags) == 0, "silu ties");
                CHECK(anchor >= 0 && anchor < n / 16, "anchor block");
                run_tensor(xb, 0, rows, cols);
            }
            free(flags);
            if (cols % 16 == 0 && cols >= 16) {
                uint8_t *kind = xmalloc((size_t)(n / 16));
                CHECK(synth_kv_heads(0, rows, cols / 16, 16, xf, kind) == 0, "kv heads");
                run_tensor(xf, 1, rows, cols);
                free(kind);
            }
        }
        CHECK(synth_gauss_outliers(0, 2, 16, 17, 1, 2, xb, NULL) == -1, "outliers: more columns than exist");
        CHECK(synth_silu_ties(0, 2, 24, 0, xb, NULL, NULL, NULL) == -1, "silu ties: bad cols");
        CHECK(synth_kv_heads(0, 2, 2, 24, xf, NULL) == -1, "kv heads: bad dim");
        free(xb);
        free(xf);
        free(d);
    }
    {
        uint8_t q[8], s[1];
        float g, a;
        uint16_t x[16] = {0};
        CHECK(oracle_quantize(x, 0, 1, 24, 1, q, s, &g, &a, 1) == -1, "bad cols rejected");
        CHECK(oracle_quantize_given_scale(x, 0, 1, 16, 1, -1.0f, q, s, 1) == -1, "bad scale rejected");
        CHECK(oracle_quantize(x, 0, 1, 16, 1, q, s, &g, &a, 1) == 0 && g == 1.0f && a == 0.0f && s[0] == 0,
              "zero tensor");
    }
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("oracle and generators clean\n");
    return 0;
}
