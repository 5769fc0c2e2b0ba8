/*
 * Host sanitizer driver for the library's C ABI (test code).  Built against a
 * compile of nvfp4rq.hip whose host code (not its device code) carries
 * AddressSanitizer and UndefinedBehaviorSanitizer, and run where no GPU is
 * visible: every entry
 * point goes through its argument validation, shape arithmetic and launch
 * planning (grid sizes, chunk counts, scale layout, head placement) up to the
 * first launch, which the runtime then rejects (NVFP4_ERR_HIP).
 *
 * Device pointers are fake addresses, 2^46 bytes apart so that even the
 * largest accepted tensor does not make two of them overlap; they are never
 * dereferenced on the host.  The program refuses to run when the runtime
 * reports a device, since a launch would then really happen with them.
 *
 * Exit status: 0 clean, 1 a status differed from the documented one, 3 a
 * device is visible (nothing called).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "nvfp4rq.h"

enum { OK = NVFP4_OK, NUL = NVFP4_ERR_NULL, SHP = NVFP4_ERR_SHAPE, ALN = NVFP4_ERR_ALIGN,
       ARG = NVFP4_ERR_ARG, HIP = NVFP4_ERR_HIP, VALID = 100 };

static int failures = 0;
static long calls = 0, rejected_launches = 0;

#define FAKE(k) ((uintptr_t)(k) << 46)

static void expect(const char *what, int64_t rows, int64_t cols, int got, int want)
{
    calls++;
    rejected_launches += got == NVFP4_ERR_HIP;
    int ok = (want == VALID) ? (got == NVFP4_OK || got == NVFP4_ERR_HIP) : got == want;
    if (!ok) {
        fprintf(stderr, "FAIL %s rows=%lld cols=%lld: status %d (%s), expected %s%d\n", what,
                (long long)rows, (long long)cols, got, nvfp4_status_string((nvfp4_status)got),
                want == VALID ? "OK or HIP, not " : "", want == VALID ? got : want);
        failures++;
    }
}

/* ------------------------------------------------ quantize-shaped entry points */

typedef struct {
    uintptr_t x, q, s, g, a;
    int64_t rows, cols;
    int rotate;
} QArgs;

typedef int (*QFn)(const QArgs *);

static int q_rotquant(const QArgs *p)
{
    return nvfp4_rotquant((const uint16_t *)p->x, p->rows, p->cols, p->rotate, (uint8_t *)p->q,
                          (uint8_t *)p->s, (float *)p->g, (float *)p->a, 0);
}
static int q_rotquant_f32(const QArgs *p)
{
    return nvfp4_rotquant_f32((const float *)p->x, p->rows, p->cols, p->rotate, (uint8_t *)p->q,
                              (uint8_t *)p->s, (float *)p->g, (float *)p->a, 0);
}
static int q_swizzled(const QArgs *p)
{
    return nvfp4_rotquant_swizzled((const uint16_t *)p->x, p->rows, p->cols, p->rotate, (uint8_t *)p->q,
                                   (uint8_t *)p->s, (float *)p->g, (float *)p->a, 0);
}
static int q_swizzled_f32(const QArgs *p)
{
    return nvfp4_rotquant_swizzled_f32((const float *)p->x, p->rows, p->cols, p->rotate, (uint8_t *)p->q,
                                       (uint8_t *)p->s, (float *)p->g, (float *)p->a, 0);
}
static int q_from_amax(const QArgs *p)
{
    return nvfp4_quant_from_amax((const uint16_t *)p->x, p->rows, p->cols, p->rotate, (const float *)p->a,
                                 (uint8_t *)p->q, (uint8_t *)p->s, (float *)p->g, 0);
}
static int q_from_amax_f32(const QArgs *p)
{
    return nvfp4_quant_from_amax_f32((const float *)p->x, p->rows, p->cols, p->rotate, (const float *)p->a,
                                     (uint8_t *)p->q, (uint8_t *)p->s, (float *)p->g, 0);
}
static int q_timed(const QArgs *p)
{
    hipEvent_t ev[6] = {0};
    int nk = -1;
    int r = nvfp4_rotquant_timed((const uint16_t *)p->x, p->rows, p->cols, p->rotate, (uint8_t *)p->q,
                                 (uint8_t *)p->s, (float *)p->g, (float *)p->a, 0, ev, 3, &nk);
    if (nk < 0 || nk > 3) {
        fprintf(stderr, "FAIL timed: nkernels %d\n", nk);
        failures++;
    }
    return r;
}
static int q_timed_f32(const QArgs *p)
{
    hipEvent_t ev[6] = {0};
    int nk = -1;
    int r = nvfp4_rotquant_f32_timed((const float *)p->x, p->rows, p->cols, p->rotate, (uint8_t *)p->q,
                                     (uint8_t *)p->s, (float *)p->g, (float *)p->a, 0, ev, 3, &nk);
    if (nk < 0 || nk > 3) {
        fprintf(stderr, "FAIL timed f32: nkernels %d\n", nk);
        failures++;
    }
    return r;
}

static const struct {
    const char *name;
    QFn fn;
    int f32, swizzled;
} QENTRIES[] = {
    {"nvfp4_rotquant", q_rotquant, 0, 0},
    {"nvfp4_rotquant_f32", q_rotquant_f32, 1, 0},
    {"nvfp4_rotquant_swizzled", q_swizzled, 0, 1},
    {"nvfp4_rotquant_swizzled_f32", q_swizzled_f32, 1, 1},
    {"nvfp4_quant_from_amax", q_from_amax, 0, 0},
    {"nvfp4_quant_from_amax_f32", q_from_amax_f32, 1, 0},
    {"nvfp4_rotquant_timed", q_timed, 0, 0},
    {"nvfp4_rotquant_f32_timed", q_timed_f32, 1, 0},
};

static void quant_validation(void)
{
    for (size_t e = 0; e < sizeof QENTRIES / sizeof QENTRIES[0]; e++) {
        const char *nm = QENTRIES[e].name;
        QFn f = QENTRIES[e].fn;
        const QArgs base = {FAKE(1), FAKE(2), FAKE(3), FAKE(4), FAKE(5), 4, 256, 1};
        QArgs a;
#define TRY(field, value, want)                      \
        do {                                         \
            a = base;                                \
            a.field = value;                         \
            expect(nm, a.rows, a.cols, f(&a), want); \
        } while (0)
        expect(nm, 4, 256, f(&base), VALID);
        TRY(x, 0, NUL);
        TRY(q, 0, NUL);
        TRY(s, 0, NUL);
        TRY(g, 0, NUL);
        TRY(a, 0, NUL);
        TRY(cols, 24, SHP);
        TRY(cols, -16, SHP);
        TRY(rows, -1, SHP);
        TRY(rows, INT64_MAX, SHP);
        TRY(rows, (int64_t)1 << 40, SHP);
        TRY(rotate, 2, ARG);
        TRY(rotate, -1, ARG);
        TRY(x, FAKE(1) + 8, ALN);
        TRY(q, FAKE(2) + 8, ALN);
        TRY(s, FAKE(3) + 2, ALN);
        TRY(g, FAKE(4) + 2, ALN);
        TRY(a, FAKE(5) + 1, ALN);
        TRY(q, FAKE(1), ARG);            /* output on the input */
        TRY(s, FAKE(2) + 16, ARG);       /* two outputs overlap */
        TRY(g, FAKE(3), ARG);
        TRY(x, FAKE(5) - 16, ARG);       /* the amax word inside the input */
        /* empty tensors: only the scalars are needed */
        a = base;
        a.rows = 0;
        a.x = a.q = a.s = 0;
        expect(nm, 0, 256, f(&a), VALID);
        a.g = 0;
        expect(nm, 0, 256, f(&a), NUL);
#undef TRY
    }
}

/* every quantize-shaped entry on shapes from one block up to the largest the
   checks accept, then just past it */
static void quant_planning(void)
{
    static const int64_t shapes[][2] = {
        {1, 16}, {3, 48}, {128, 1024}, {129, 1040}, {4096, 4096}, {16384, 8192}, {32768, 14336},
        {65536, 1024}, {524288, 128}, {1, 1 << 20}, {1 << 22, 16}, {1 << 20, 1 << 15},
        {((int64_t)1 << 31) - 1, 4096}, {(int64_t)1 << 31, 4096}, {(int64_t)1 << 27, (int64_t)1 << 16},
        {1, ((int64_t)1 << 43) - 16}, {1, (int64_t)1 << 43}, {2, (int64_t)1 << 22}, {130, (int64_t)1 << 23},
    };
    for (size_t e = 0; e < sizeof QENTRIES / sizeof QENTRIES[0]; e++) {
        for (size_t t = 0; t < sizeof shapes / sizeof shapes[0]; t++) {
            const int64_t rows = shapes[t][0], cols = shapes[t][1];
            const int64_t nb = rows * (cols / 16);
            int want = nb < ((int64_t)1 << 39) ? VALID : SHP;
            if (QENTRIES[e].swizzled) {
                const int64_t lim = ((int64_t)1 << 31) / (128 * (QENTRIES[e].f32 ? 4 : 2));
                if (nb > 0xFFFFFFFFLL || cols >= lim)
                    want = SHP;
            }
            for (int rot = 0; rot < 2; rot++) {
                QArgs a = {FAKE(1), FAKE(2), FAKE(3), FAKE(4), FAKE(5), rows, cols, rot};
                expect(QENTRIES[e].name, rows, cols, QENTRIES[e].fn(&a), want);
            }
        }
    }
}

/* ------------------------------------------------------ the other entry points */

static void other_entries(void)
{
    const uint16_t *xb = (const uint16_t *)FAKE(1);
    const float *xf = (const float *)FAKE(1);
    uint8_t *q = (uint8_t *)FAKE(2), *s = (uint8_t *)FAKE(3);
    float *g = (float *)FAKE(4), *a = (float *)FAKE(5), *y = (float *)FAKE(6);
    const float *r16 = (const float *)FAKE(7);

    /* amax alone */
    expect("rotamax", 4, 64, nvfp4_rotamax(xb, 4, 64, 1, a, 0), VALID);
    expect("rotamax_f32", 4, 64, nvfp4_rotamax_f32(xf, 4, 64, 0, a, 0), VALID);
    expect("rotamax", 4, 64, nvfp4_rotamax(NULL, 4, 64, 1, a, 0), NUL);
    expect("rotamax", 4, 64, nvfp4_rotamax(xb, 4, 64, 1, NULL, 0), NUL);
    expect("rotamax", 4, 40, nvfp4_rotamax(xb, 4, 40, 1, a, 0), SHP);
    expect("rotamax", 4, 64, nvfp4_rotamax(xb, 4, 64, 3, a, 0), ARG);
    expect("rotamax", 4, 64, nvfp4_rotamax(xb + 4, 4, 64, 1, a, 0), ALN);
    expect("rotamax", 4, 64, nvfp4_rotamax(xb, 4, 64, 1, (float *)((uintptr_t)a + 2), 0), ALN);
    expect("rotamax", 4, 64, nvfp4_rotamax(xb, 4, 64, 1, (float *)(xb + 32), 0), ARG);
    expect("rotamax", 0, 64, nvfp4_rotamax(NULL, 0, 64, 1, a, 0), VALID);
    expect("rotamax", 1 << 20, 1 << 15, nvfp4_rotamax(xb, 1 << 20, 1 << 15, 1, a, 0), VALID);
    expect("rotamax_f32", 1 << 20, 1 << 15, nvfp4_rotamax_f32(xf, 1 << 20, 1 << 15, 1, a, 0), VALID);

    /* dequantize, both scale layouts */
    expect("dequant", 4, 64, nvfp4_dequant(q, s, g, 4, 64, 1, y, 0), VALID);
    expect("dequant", 4, 64, nvfp4_dequant(NULL, s, g, 4, 64, 1, y, 0), NUL);
    expect("dequant", 4, 64, nvfp4_dequant(q, NULL, g, 4, 64, 1, y, 0), NUL);
    expect("dequant", 4, 64, nvfp4_dequant(q, s, NULL, 4, 64, 1, y, 0), NUL);
    expect("dequant", 4, 64, nvfp4_dequant(q, s, g, 4, 64, 1, NULL, 0), NUL);
    expect("dequant", 4, 56, nvfp4_dequant(q, s, g, 4, 56, 1, y, 0), SHP);
    expect("dequant", 4, 64, nvfp4_dequant(q, s, g, 4, 64, 7, y, 0), ARG);
    expect("dequant", 4, 64, nvfp4_dequant(q + 4, s, g, 4, 64, 1, y, 0), ALN);
    expect("dequant", 4, 64, nvfp4_dequant(q, s, g, 4, 64, 1, y + 2, 0), ALN);
    expect("dequant", 4, 64, nvfp4_dequant(q, s, g, 4, 64, 1, (float *)q, 0), ARG);
    expect("dequant", 1 << 20, 1 << 15, nvfp4_dequant(q, s, g, 1 << 20, 1 << 15, 0, y, 0), VALID);
    expect("dequant_swizzled", 4, 64, nvfp4_dequant_swizzled(q, s, g, 4, 64, 1, y, 0), VALID);
    expect("dequant_swizzled", 300, 1040, nvfp4_dequant_swizzled(q, s, g, 300, 1040, 0, y, 0), VALID);
    expect("dequant_swizzled", 4, 64, nvfp4_dequant_swizzled(q, s, NULL, 4, 64, 1, y, 0), NUL);
    expect("dequant_swizzled", 4, 48 + 8, nvfp4_dequant_swizzled(q, s, g, 4, 56, 1, y, 0), SHP);

    /* swizzled scale sizes */
    calls++;
    if (nvfp4_swizzled_scale_bytes(1, 16) != 512 || nvfp4_swizzled_scale_bytes(129, 80) != 2 * 2 * 512 ||
        nvfp4_swizzled_scale_bytes(0, 64) != 0 || nvfp4_swizzled_scale_bytes(4, 24) != -1 ||
        nvfp4_swizzled_scale_bytes(-1, 16) != -1 || nvfp4_swizzled_scale_bytes(INT64_MAX, 16) != -1 ||
        nvfp4_swizzled_scale_bytes((int64_t)1 << 33, 16) != -1) {
        fprintf(stderr, "FAIL nvfp4_swizzled_scale_bytes\n");
        failures++;
    }

    /* rotation alone, and the general 16 x 16 rotation */
    expect("rotate16", 4, 64, nvfp4_rotate16(xb, 4, 64, y, 0), VALID);
    expect("rotate16_f32", 4, 64, nvfp4_rotate16_f32(xf, 4, 64, y, 0), VALID);
    expect("rotate16", 4, 64, nvfp4_rotate16(NULL, 4, 64, y, 0), NUL);
    expect("rotate16", 4, 64, nvfp4_rotate16(xb, 4, 64, (float *)xb, 0), ARG);
    expect("rotate16", 4, 64, nvfp4_rotate16(xb, 4, 64, y + 1, 0), ALN);
    expect("rotate16", 1 << 20, 1 << 15, nvfp4_rotate16(xb, 1 << 20, 1 << 15, y, 0), VALID);
    expect("rotate_matrix", 4, 64, nvfp4_rotate_matrix(xb, 4, 64, r16, y, 0), VALID);
    expect("rotate_matrix_f32", 4, 64, nvfp4_rotate_matrix_f32(xf, 4, 64, r16, y, 0), VALID);
    expect("rotate_matrix", 4, 64, nvfp4_rotate_matrix(xb, 4, 64, NULL, y, 0), NUL);
    expect("rotate_matrix", 0, 64, nvfp4_rotate_matrix(NULL, 0, 64, NULL, NULL, 0), NUL);
    expect("rotate_matrix", 0, 64, nvfp4_rotate_matrix(NULL, 0, 64, r16, NULL, 0), OK);
    expect("rotate_matrix", 4, 64, nvfp4_rotate_matrix(xb, 4, 64, r16 + 2, y, 0), ALN);
    expect("rotate_matrix", 4, 64, nvfp4_rotate_matrix(xb, 4, 64, (const float *)y, y, 0), ARG);

    /* MXFP4 */
    expect("mxfp4_rotquant", 4, 64, mxfp4_rotquant(xb, 4, 64, 1, q, s, 0), VALID);
    expect("mxfp4_rotquant_f32", 4, 64, mxfp4_rotquant_f32(xf, 4, 64, 0, q, s, 0), VALID);
    expect("mxfp4_rotquant", 4, 48, mxfp4_rotquant(xb, 4, 48, 1, q, s, 0), SHP);
    expect("mxfp4_rotquant", 4, 64, mxfp4_rotquant(xb, 4, 64, 1, NULL, s, 0), NUL);
    expect("mxfp4_rotquant", 4, 64, mxfp4_rotquant(xb, 4, 64, 5, q, s, 0), ARG);
    expect("mxfp4_rotquant", 4, 64, mxfp4_rotquant(xb, 4, 64, 1, q + 8, s, 0), ALN);
    expect("mxfp4_rotquant", 4, 64, mxfp4_rotquant(xb, 4, 64, 1, q, q + 16, 0), ARG);
    expect("mxfp4_rotquant", 1 << 20, 1 << 15, mxfp4_rotquant(xb, 1 << 20, 1 << 15, 1, q, s, 0), VALID);
    expect("mxfp4_dequant", 4, 64, mxfp4_dequant(q, s, 4, 64, 1, y, 0), VALID);
    expect("mxfp4_dequant", 4, 48, mxfp4_dequant(q, s, 4, 48, 1, y, 0), SHP);
    expect("mxfp4_dequant", 4, 64, mxfp4_dequant(q, s, 4, 64, 1, NULL, 0), NUL);

    /* the calibration stream */
    expect("stream_calibrate", 4, 64, nvfp4_stream_calibrate(xb, 4, 64, q, s, 0), VALID);
    expect("stream_calibrate_f32", 4, 64, nvfp4_stream_calibrate_f32(xf, 4, 64, q, s, 0), VALID);
    expect("stream_calibrate", 4, 64, nvfp4_stream_calibrate(NULL, 4, 64, q, s, 0), NUL);
    expect("stream_calibrate", 4, 40, nvfp4_stream_calibrate(xb, 4, 40, q, s, 0), SHP);
    expect("stream_calibrate_single", 4, 64, nvfp4_stream_calibrate_single(xb, 4, 64, q, s, 0), VALID);
    expect("stream_calibrate_single_f32", 4, 64, nvfp4_stream_calibrate_single_f32(xf, 4, 64, q, s, 0), VALID);
    expect("stream_calibrate_single", 4, 64, nvfp4_stream_calibrate_single(NULL, 4, 64, q, s, 0), NUL);
    expect("stream_calibrate_single", 4, 40, nvfp4_stream_calibrate_single(xb, 4, 40, q, s, 0), SHP);
    expect("stream_calibrate", 4, 64, nvfp4_stream_calibrate(xb + 4, 4, 64, q, s, 0), ALN);
    expect("stream_calibrate", 4, 64, nvfp4_stream_calibrate(xb, 4, 64, (uint8_t *)xb, s, 0), ARG);
    expect("stream_calibrate", 16384, 8192, nvfp4_stream_calibrate(xb, 16384, 8192, q, s, 0), VALID);
    expect("stream_calibrate", 1 << 20, 1 << 15, nvfp4_stream_calibrate(xb, 1 << 20, 1 << 15, q, s, 0), VALID);

    /* the timing variants' own arguments */
    int nk = 0;
    hipEvent_t ev[2] = {0};
    expect("rotquant_timed", 4, 64,
           nvfp4_rotquant_timed(xb, 4, 64, 1, q, s, g, a, 0, NULL, 1, &nk), NUL);
    expect("rotquant_timed", 4, 64, nvfp4_rotquant_timed(xb, 4, 64, 1, q, s, g, a, 0, ev, 0, &nk), NUL);
    expect("rotquant_timed", 4, 64, nvfp4_rotquant_timed(xb, 4, 64, 1, q, s, g, a, 0, ev, 1, NULL), NUL);

    /* status text, including codes outside the enum */
    for (int c = -2; c < 8; c++) {
        calls++;
        const char *t = nvfp4_status_string((nvfp4_status)c);
        if (!t || !*t) {
            fprintf(stderr, "FAIL status string %d\n", c);
            failures++;
        }
    }
}

int main(void)
{
    int n = -1;
    const hipError_t e = hipGetDeviceCount(&n);
    if (e == hipSuccess && n > 0) {
        fprintf(stderr, "a device is visible: this driver only runs without one\n");
        return 3;
    }
    quant_validation();
    quant_planning();
    other_entries();
    if (failures) {
        fprintf(stderr, "%d of %ld checks failed\n", failures, calls);
        return 1;
    }
    printf("C ABI clean under the host sanitizers: %ld checks, %ld reached a launch\n", calls,
           rejected_launches);
    return 0;
}
