/*
 * CPU oracle for fused block-Hadamard rotation + NVFP4 activation quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry and the
 * benchmark's CPU-baseline leg may load this library.  The product path never
 * links, loads or calls it, and it shares no code, header, table or constant
 * generator with the HIP library.
 *
 * What it computes follows the page "A Fused Hadamard + NVFP4 Quantization
 * Kernel in Triton" (kanthi.in): section 1 "The format, precisely" fixes the
 * two-level scaling, section 2 "The kernel" fixes the arithmetic (fp32 block
 * rotation, global scale from the rotated amax, explicitly rounded E4M3 block
 * scale, divide, E2M1 thresholds, nibble packing) and section 3 "Bit-exact
 * against a reference" restates the same arithmetic with PyTorch's
 * round-to-nearest-even E4M3 cast.  The stored layout (two nibbles per byte,
 * one E4M3 byte per 16 values along K) also matches the page "NVFP4
 * Quantization" (atlas-docs), section "The numeric format".
 *
 * Style: plain scalar C, one block at a time, every floating-point operation a
 * single IEEE-754 binary32 operation in round-to-nearest-even, in the order the
 * definition states.  Build with -O2 -ffp-contract=off and without
 * -ffast-math; x86-64 evaluates float expressions in binary32 (SSE), so each
 * C operator below is exactly one rounding.  OpenMP only splits independent
 * rows; a maximum is exact and order-free, so the thread count never changes a
 * byte.
 *
 * Readings where the page is silent or contradicts itself (each one is listed
 * with its reason in the design notes):
 *   - rotation order: iterative butterfly, strides 1, 2, 4, 8, pairs
 *     (a+b, a-b), then a final multiply by 0.25;
 *   - global scale: (amax / 6) / 448, two binary32 divisions, 1.0 when zero;
 *   - block scale: (block_amax / 6) / g, then round to nearest E4M3 with ties
 *     to even mantissa, E4M3 subnormals kept, clamped at 448;
 *   - element quotient: one IEEE binary32 division per element;
 *   - E2M1 code: alternating > / >= midpoint compares (ties to the even code),
 *     sign bit set only when the quotient compares below zero (-0.0 -> 0);
 *   - no flush-to-zero anywhere.
 *
 * Parity pins: every function here is pinned by a CPU test against something
 * other than itself (tables and worked values printed on the page, exhaustive
 * sweeps against nearest-point searches, PyTorch's float8 cast, an
 * exact-rational re-implementation, closed forms).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* element helpers                                                      */
/* ------------------------------------------------------------------ */

/* bf16 is the top half of a binary32; widening is exact. */
static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * Block rotation y = x * H16 with H16 the 16x16 Sylvester-Hadamard matrix
 * scaled by 1/4 (section 1: orthonormal, H*H^T = I; section 2, hadamard16:
 * Kronecker doubling [[H, H], [H, -H]] four times, then /4).
 * H16 is symmetric, so x*H16 == H16*x.  The fast transform below applies the
 * four doublings as butterfly stages with strides 1, 2, 4, 8 (each stage
 * replaces a pair (a, b) with (a+b, a-b)), then scales by 0.25.
 */
void oracle_rotate16(const float *x, float *y)
{
    float z[16];
    for (int i = 0; i < 16; i++)
        z[i] = x[i];
    for (int h = 1; h < 16; h *= 2) {
        for (int i = 0; i < 16; i++) {
            if ((i & h) == 0) {
                float a = z[i];
                float b = z[i + h];
                z[i] = a + b;
                z[i + h] = a - b;
            }
        }
    }
    for (int i = 0; i < 16; i++)
        y[i] = 0.25f * z[i];
}

/*
 * E2M1 element code (section 2, _e2m1_code; section 3, reference): the
 * magnitude index is the number of the seven grid midpoints
 * 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0 that |v| passes, where the comparison
 * alternates between strict and non-strict so that an exact midpoint goes to
 * the neighbour with even code (0, 1.0, 2.0, 4.0).  Bit 3 is set when v < 0.
 */
uint8_t oracle_e2m1_code(float v)
{
    float a = fabsf(v);
    int m = 0;
    if (a > 0.25f) m++;
    if (a >= 0.75f) m++;
    if (a > 1.25f) m++;
    if (a >= 1.75f) m++;
    if (a > 2.5f) m++;
    if (a >= 3.5f) m++;
    if (a > 5.0f) m++;
    if (v < 0.0f) m += 8;
    return (uint8_t)m;
}

/* Magnitude of an E2M1 code's grid point: {0, .5, 1, 1.5, 2, 3, 4, 6}
 * (section 1 table; section 2, dequantize's GRID). */
static const double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/*
 * Value of a non-negative E4M3FN byte 0x00..0x7E: 4 exponent bits with bias 7,
 * 3 mantissa bits, exponent field 0 holding the subnormals k * 2^-9.
 * (section 1: E4M3 block scale, maximum 448 = 0x7E.)
 */
float oracle_e4m3_value(uint8_t b)
{
    int e = (b >> 3) & 15;
    int m = b & 7;
    if (e == 0)
        return ldexpf((float)m, -9);
    return ldexpf(1.0f + (float)m / 8.0f, e - 7);
}

/*
 * Round a non-negative binary32 to the E4M3 grid and return the byte
 * (section 2, _round_e4m3: exponent of the value clamped below at -6, step
 * 2^(e-3), round v/step to an integer, clamp at 448; section 3 uses the
 * round-to-nearest-even cast).  Reading: ties go to the even mantissa, as
 * PyTorch's cast does, and the exponent comes from the float's own exponent
 * field (frexpf), never from a logarithm.  v/step and the products below are
 * scalings by powers of two and therefore exact.
 */
uint8_t oracle_e4m3_byte(float v)
{
    if (!(v > 0.0f))
        return 0;                 /* +0 (negative input is outside the contract) */
    if (v >= 448.0f)
        return 0x7E;              /* min(round(v), 448) is 448 for every v >= 448 */
    int fe;
    (void)frexpf(v, &fe);         /* v = f * 2^fe, f in [0.5, 1) */
    int e = fe - 1;               /* v = (2f) * 2^e, 2f in [1, 2) */
    if (e < -6)
        e = -6;                   /* below the smallest normal the step stays 2^-9 */
    float k = ldexpf(v, 3 - e);   /* v / 2^(e-3), exact */
    float kf = floorf(k);
    float frac = k - kf;          /* exact: k < 16 has at most 4 integer bits */
    int ki = (int)kf;
    if (frac > 0.5f || (frac == 0.5f && (ki & 1)))
        ki++;                     /* nearest integer, ties to even */
    /* ki in 0..16; the byte is exponent field (e+7) and mantissa ki-8, with the
       carry of ki == 16 moving into the exponent field by itself. */
    return (uint8_t)(((e + 7) << 3) + ki - 8);
}

/*
 * Global scale s_global = amax / (448 * 6) (section 1), computed as the code of
 * section 2 (quantize) and section 3 (reference) does: divide by 6.0, then by
 * 448.0, each in binary32, and use 1.0 when the result is zero.
 */
float oracle_global_scale(float amax)
{
    float g = (amax / 6.0f) / 448.0f;
    if (g == 0.0f)
        g = 1.0f;
    return g;
}

/* ------------------------------------------------------------------ */
/* tensor passes                                                        */
/* ------------------------------------------------------------------ */

static void load_block(const void *x, int is_f32, int64_t b, float *out)
{
    if (is_f32) {
        const float *p = (const float *)x + b * 16;
        for (int i = 0; i < 16; i++)
            out[i] = p[i];
    } else {
        const uint16_t *p = (const uint16_t *)x + b * 16;
        for (int i = 0; i < 16; i++)
            out[i] = bf16_to_float(p[i]);
    }
}

/* The values a block is scaled from: rotated when `rotate`, else as loaded. */
static void block_values(const void *x, int is_f32, int rotate, int64_t b, float *y)
{
    float xb[16];
    load_block(x, is_f32, b, xb);
    if (rotate)
        oracle_rotate16(xb, y);
    else
        for (int i = 0; i < 16; i++)
            y[i] = xb[i];
}

/*
 * Pass 1: the largest |y| over the whole (rotated) tensor (section 2, quantize:
 * the wrapper takes this maximum first, since every block scale depends on
 * it).  Block b covers elements 16b .. 16b+15 of the row-major tensor,
 * which is a reshape to [-1, 16]; with cols % 16 == 0 no block crosses a row.
 */
float oracle_amax(const void *x, int is_f32, int64_t rows, int64_t cols, int rotate,
                  int nthreads)
{
    int64_t nb = rows * (cols / 16);
    float amax = 0.0f;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) reduction(max : amax) schedule(static)
#endif
    for (int64_t b = 0; b < nb; b++) {
        float y[16];
        block_values(x, is_f32, rotate, b, y);
        for (int i = 0; i < 16; i++) {
            float a = fabsf(y[i]);
            if (a > amax)
                amax = a;
        }
    }
    (void)nthreads;
    return amax;
}

/*
 * Pass 2 for one block (section 2, hadamard_nvfp4_kernel; section 3,
 * reference):
 *   a_b = max |y_i|
 *   s   = E4M3(min(round((a_b / 6) / g), 448))
 *   sf  = float(s) * g ; divisor d = 1.0 when sf == 0, else sf
 *   v_i = y_i / d       (binary32 division)
 *   code_i = E2M1 code of v_i
 *   q[k] = code[2k] | code[2k+1] << 4   (even element in the low nibble)
 */
static void quantize_block(const float *y, float g, uint8_t *q8, uint8_t *s1)
{
    float ab = 0.0f;
    for (int i = 0; i < 16; i++) {
        float a = fabsf(y[i]);
        if (a > ab)
            ab = a;
    }
    float v = (ab / 6.0f) / g;
    uint8_t s = oracle_e4m3_byte(v);
    float sf = oracle_e4m3_value(s) * g;
    float d = (sf == 0.0f) ? 1.0f : sf;
    uint8_t code[16];
    for (int i = 0; i < 16; i++)
        code[i] = oracle_e2m1_code(y[i] / d);
    for (int k = 0; k < 8; k++)
        q8[k] = (uint8_t)(code[2 * k] | (code[2 * k + 1] << 4));
    *s1 = s;
}

/*
 * The whole method: pass 1 (global rotated amax), the global scale, then every
 * block quantized with it.  Outputs: q [rows, cols/2] packed codes, s
 * [rows, cols/16] E4M3 bytes, *g_out the global scale, *amax_out the amax.
 * Returns 0, or -1 when cols is not a multiple of 16.
 */
int oracle_quantize(const void *x, int is_f32, int64_t rows, int64_t cols, int rotate,
                    uint8_t *q, uint8_t *s, float *g_out, float *amax_out, int nthreads)
{
    if (cols % 16 != 0 || rows < 0 || cols < 0)
        return -1;
    float amax = oracle_amax(x, is_f32, rows, cols, rotate, nthreads);
    float g = oracle_global_scale(amax);
    int64_t nb = rows * (cols / 16);
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(static)
#endif
    for (int64_t b = 0; b < nb; b++) {
        float y[16];
        block_values(x, is_f32, rotate, b, y);
        quantize_block(y, g, q + 8 * b, s + b);
    }
    *g_out = g;
    *amax_out = amax;
    return 0;
}

/*
 * Quantize with a global scale supplied by the caller (section 2 notes that a
 * production stack may reuse an amax from an earlier step): the same block
 * arithmetic, no amax pass.  The clamp at 448 becomes reachable here.
 */
int oracle_quantize_given_scale(const void *x, int is_f32, int64_t rows, int64_t cols,
                                int rotate, float g, uint8_t *q, uint8_t *s, int nthreads)
{
    if (cols % 16 != 0 || rows < 0 || cols < 0 || !(g > 0.0f))
        return -1;
    int64_t nb = rows * (cols / 16);
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(static)
#endif
    for (int64_t b = 0; b < nb; b++) {
        float y[16];
        block_values(x, is_f32, rotate, b, y);
        quantize_block(y, g, q + 8 * b, s + b);
    }
    (void)nthreads;
    return 0;
}

/* ------------------------------------------------------------------ */
/* dequantization and round-trip error (fp64)                          */
/* ------------------------------------------------------------------ */

/*
 * Decode one block back to the input space (section 2, dequantize): each code
 * becomes +-GRID[code & 7], times float(s) * g, each product rounded to
 * binary32 as the page's fp32 tensors do; then, when rotated, multiplied by
 * H16^T = H16, here in fp64 with the exact matrix entries (-1)^popcount(i&j)/4.
 */
static void dequant_block(const uint8_t *q8, uint8_t s, float g, int rotate, double *out)
{
    float sf = oracle_e4m3_value(s) * g;
    double yh[16];
    for (int i = 0; i < 16; i++) {
        int c = (i & 1) ? (q8[i / 2] >> 4) : (q8[i / 2] & 15);
        float mag = (float)E2M1_GRID[c & 7];
        float val = (c & 8) ? -mag : mag;
        yh[i] = (double)(val * sf);
    }
    if (!rotate) {
        for (int i = 0; i < 16; i++)
            out[i] = yh[i];
        return;
    }
    for (int i = 0; i < 16; i++) {
        double acc = 0.0;
        for (int j = 0; j < 16; j++) {
            int sign = __builtin_popcount((unsigned)(i & j)) & 1;
            acc += (sign ? -yh[j] : yh[j]) * 0.25;
        }
        out[i] = acc;
    }
}

/* Dequantize a whole tensor into fp64 [rows, cols]. */
void oracle_dequant_f64(const uint8_t *q, const uint8_t *s, float g, int64_t rows,
                        int64_t cols, int rotate, double *out, int nthreads)
{
    int64_t nb = rows * (cols / 16);
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(static)
#endif
    for (int64_t b = 0; b < nb; b++)
        dequant_block(q + 8 * b, s[b], g, rotate, out + 16 * b);
    (void)nthreads;
}

/*
 * Relative L2 round-trip error ||x_hat - x|| / ||x|| with sums in fp64
 * (section 3, run_demo; section 5, error_study).  When col_mask is not NULL,
 * only columns with col_mask[c] != 0 enter both norms (section 5's "normal
 * columns" case).  Returns NaN for an all-zero x.
 */
double oracle_roundtrip_error(const void *x, int is_f32, int64_t rows, int64_t cols,
                              int rotate, const uint8_t *q, const uint8_t *s, float g,
                              const uint8_t *col_mask, int nthreads)
{
    int64_t nb = rows * (cols / 16);
    int64_t bpr = cols / 16;
    double num = 0.0, den = 0.0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) reduction(+ : num, den) schedule(static)
#endif
    for (int64_t b = 0; b < nb; b++) {
        float xb[16];
        double xh[16];
        load_block(x, is_f32, b, xb);
        dequant_block(q + 8 * b, s[b], g, rotate, xh);
        int64_t c0 = (b % bpr) * 16;
        for (int i = 0; i < 16; i++) {
            if (col_mask && !col_mask[c0 + i])
                continue;
            double d = xh[i] - (double)xb[i];
            num += d * d;
            den += (double)xb[i] * (double)xb[i];
        }
    }
    (void)nthreads;
    return sqrt(num) / sqrt(den);
}

/* ------------------------------------------------------------------ */
/* array forms of the element helpers, for exhaustive sweeps            */
/* ------------------------------------------------------------------ */

void oracle_e2m1_code_array(const float *v, int64_t n, uint8_t *out, int nthreads)
{
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(static)
#endif
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_e2m1_code(v[i]);
    (void)nthreads;
}

void oracle_e4m3_byte_array(const float *v, int64_t n, uint8_t *out, int nthreads)
{
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(static)
#endif
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_e4m3_byte(v[i]);
    (void)nthreads;
}

/* Codes for every binary32 bit pattern in [lo, hi] (inclusive), for sweeps. */
void oracle_e2m1_code_bits(uint32_t lo, uint32_t hi, uint8_t *out, int nthreads)
{
    int64_t n = (int64_t)hi - (int64_t)lo + 1;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(static)
#endif
    for (int64_t i = 0; i < n; i++) {
        uint32_t u = lo + (uint32_t)i;
        float f;
        memcpy(&f, &u, sizeof f);
        out[i] = oracle_e2m1_code(f);
    }
    (void)nthreads;
}

void oracle_e4m3_byte_bits(uint32_t lo, uint32_t hi, uint8_t *out, int nthreads)
{
    int64_t n = (int64_t)hi - (int64_t)lo + 1;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(static)
#endif
    for (int64_t i = 0; i < n; i++) {
        uint32_t u = lo + (uint32_t)i;
        float f;
        memcpy(&f, &u, sizeof f);
        out[i] = oracle_e4m3_byte(f);
    }
    (void)nthreads;
}

/* ------------------------------------------------------------------ */
/* MXFP4 variant: 32-element blocks, power-of-two (E8M0) scales        */
/* ------------------------------------------------------------------ */

/*
 * The page "A Fused Hadamard + NVFP4 Quantization Kernel in Triton" contrasts
 * NVFP4 with MXFP4 (section 1: 32-element blocks, power-of-two E8M0 scales;
 * its "Try this" list asks for the error study under MXFP4 semantics).  The
 * page "Hopper kernel for MXFP4" stores each MX scale as one unsigned byte
 * holding a binary exponent (value 2^(byte - 127)).  Readings where the pages
 * stop short:
 *   - the rotation stays the 16-point block rotation, applied to each half of
 *     a 32-element block;
 *   - the block value is fl(amax / 6) as in the NVFP4 recipe, and the scale is
 *     the smallest power of two at or above it, so the block's largest value
 *     maps into (3, 6] (never clipped), exponent clamped to [-127, 127];
 *     an all-zero block gets the byte 0;
 *   - element values v = fl(y / scale) (an exact power-of-two scaling except
 *     on underflow), then the same E2M1 midpoint rule and sign rule;
 *   - storage: codes [rows, cols/2] as for NVFP4, scales [rows, cols/32].
 */
uint8_t oracle_e8m0_byte(float t)
{
    if (!(t > 0.0f))
        return 0;
    int fe;
    float m = frexpf(t, &fe);      /* t = m * 2^fe, m in [0.5, 1) */
    int e = (m == 0.5f) ? fe - 1 : fe;   /* ceil(log2 t) */
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return (uint8_t)(e + 127);
}

float oracle_e8m0_value(uint8_t b)
{
    return ldexpf(1.0f, (int)b - 127);
}

static void load_span(const void *x, int is_f32, int64_t start, int n, float *out)
{
    if (is_f32) {
        const float *p = (const float *)x + start;
        for (int i = 0; i < n; i++)
            out[i] = p[i];
    } else {
        const uint16_t *p = (const uint16_t *)x + start;
        for (int i = 0; i < n; i++)
            out[i] = bf16_to_float(p[i]);
    }
}

/* One 32-element MX block: optional rotation of each half, E8M0 scale, codes. */
static void mx_block(const float *xb, int rotate, uint8_t *q16, uint8_t *s1)
{
    float y[32];
    if (rotate) {
        oracle_rotate16(xb, y);
        oracle_rotate16(xb + 16, y + 16);
    } else {
        for (int i = 0; i < 32; i++)
            y[i] = xb[i];
    }
    float ab = 0.0f;
    for (int i = 0; i < 32; i++) {
        float a = fabsf(y[i]);
        if (a > ab)
            ab = a;
    }
    uint8_t s = oracle_e8m0_byte(ab / 6.0f);
    float scale = oracle_e8m0_value(s);
    uint8_t code[32];
    for (int i = 0; i < 32; i++)
        code[i] = oracle_e2m1_code(y[i] / scale);
    for (int k = 0; k < 16; k++)
        q16[k] = (uint8_t)(code[2 * k] | (code[2 * k + 1] << 4));
    *s1 = s;
}

/* MXFP4 quantization of a [rows, cols] tensor, cols % 32 == 0.  Returns 0, or
   -1 on a bad shape. */
int oracle_mx_quantize(const void *x, int is_f32, int64_t rows, int64_t cols, int rotate,
                       uint8_t *q, uint8_t *s, int nthreads)
{
    if (cols % 32 != 0 || rows < 0 || cols < 0)
        return -1;
    int64_t nb = rows * (cols / 32);
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(static)
#endif
    for (int64_t b = 0; b < nb; b++) {
        float xb[32];
        load_span(x, is_f32, b * 32, 32, xb);
        mx_block(xb, rotate, q + 16 * b, s + b);
    }
    (void)nthreads;
    return 0;
}

/* Decode of one MX block to fp64: +-GRID[c & 7] * scale (exact), then the exact
   inverse rotation H16 / 4 of each half (H16 is its own inverse up to 1/16). */
static void mx_decode_block(const uint8_t *q16, uint8_t sb, int rotate, double *out)
{
    double scale = (double)oracle_e8m0_value(sb);
    double yh[32];
    for (int i = 0; i < 32; i++) {
        int c = (i & 1) ? (q16[i / 2] >> 4) : (q16[i / 2] & 15);
        double mag = E2M1_GRID[c & 7] * scale;
        yh[i] = (c & 8) ? -mag : mag;
    }
    for (int h = 0; h < 2; h++) {
        for (int i = 0; i < 16; i++) {
            if (!rotate) {
                out[16 * h + i] = yh[16 * h + i];
                continue;
            }
            double acc = 0.0;
            for (int j = 0; j < 16; j++) {
                int sign = __builtin_popcount((unsigned)(i & j)) & 1;
                acc += (sign ? -yh[16 * h + j] : yh[16 * h + j]) * 0.25;
            }
            out[16 * h + i] = acc;
        }
    }
}

/* fp64 decode of a whole MXFP4 tensor into out [rows, cols]. */
void oracle_mx_dequant_f64(const uint8_t *q, const uint8_t *s, int64_t rows, int64_t cols,
                           int rotate, double *out, int nthreads)
{
    int64_t nb = rows * (cols / 32);
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(static)
#endif
    for (int64_t b = 0; b < nb; b++)
        mx_decode_block(q + 16 * b, s[b], rotate, out + 32 * b);
    (void)nthreads;
}

/* Relative L2 round-trip error of an MXFP4 encoding (fp64 sums, exact H). */
double oracle_mx_roundtrip_error(const void *x, int is_f32, int64_t rows, int64_t cols,
                                 int rotate, const uint8_t *q, const uint8_t *s, int nthreads)
{
    int64_t nb = rows * (cols / 32);
    double num = 0.0, den = 0.0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) reduction(+ : num, den) schedule(static)
#endif
    for (int64_t b = 0; b < nb; b++) {
        float xb[32];
        load_span(x, is_f32, b * 32, 32, xb);
        double xh[32];
        mx_decode_block(q + 16 * b, s[b], rotate, xh);
        for (int i = 0; i < 32; i++) {
            double d = xh[i] - (double)xb[i];
            num += d * d;
            den += (double)xb[i] * (double)xb[i];
        }
    }
    (void)nthreads;
    return sqrt(num) / sqrt(den);
}

/* ------------------------------------------------------------------ */
/* Rotation of a whole tensor (the first kernel of the unfused        */
/* three-kernel arrangement)                                          */
/* ------------------------------------------------------------------ */

/* y [rows, cols] fp32 = oracle_rotate16 of every 16-element block of x.
   Returns 0, or -1 on a bad shape. */
int oracle_rotate_tensor(const void *x, int is_f32, int64_t rows, int64_t cols, float *y,
                         int nthreads)
{
    if (cols % 16 != 0 || rows < 0 || cols < 0)
        return -1;
    int64_t nb = rows * (cols / 16);
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(static)
#endif
    for (int64_t b = 0; b < nb; b++) {
        float xb[16];
        load_span(x, is_f32, b * 16, 16, xb);
        oracle_rotate16(xb, y + 16 * b);
    }
    (void)nthreads;
    return 0;
}

/*
 * A general 16x16 block rotation (page "A Fused Hadamard + NVFP4
 * Quantization Kernel in Triton", "Try this" item 3: the Hadamard replaced by
 * a random orthogonal 16x16 matrix).  For each 16-element block x,
 * y_j = sum_k x_k r[k][j] (r row-major, y = x r), in binary32 with this
 * summation order, a reading the page leaves open (its tl.dot fixes none):
 * acc = RN(x_0 r[0][j]), then acc = RN(x_k r[k][j] + acc) as one fused
 * multiply-add for k = 1..15.  The same order on the GPU gives the same bits.
 * Returns 0, or -1 on a bad shape.
 */
int oracle_rotate_matrix(const void *x, int is_f32, int64_t rows, int64_t cols,
                         const float *r, float *y, int nthreads)
{
    if (cols % 16 != 0 || rows < 0 || cols < 0)
        return -1;
    int64_t nb = rows * (cols / 16);
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(static)
#endif
    for (int64_t b = 0; b < nb; b++) {
        float xb[16];
        load_span(x, is_f32, b * 16, 16, xb);
        for (int j = 0; j < 16; j++) {
            float acc = xb[0] * r[j];
            for (int k = 1; k < 16; k++)
                acc = fmaf(xb[k], r[16 * k + j], acc);
            y[16 * b + j] = acc;
        }
    }
    (void)nthreads;
    return 0;
}

/* ------------------------------------------------------------------ */
/* Swizzled block-scale layout                                        */
/* ------------------------------------------------------------------ */

/*
 * The page "A Fused Hadamard + NVFP4 Quantization Kernel in Triton", section 6
 * ("Layout"), says NVFP4 GEMMs read block scales in a swizzled tiled layout
 * rather than the row-major [rows, cols/16] matrix, and that a production
 * kernel writes that layout directly; it does not spell the layout out.
 * Reading taken: the tiled layout of the GEMM library documentation the page
 * cites for 16-element block scales.  The scale matrix S [rows, cb] (cb =
 * cols / 16) is padded with zero bytes to multiples of 128 rows and 4
 * columns and cut into 128 x 4 tiles of 512 bytes, stored tile-row by
 * tile-row (tile (rt, ct) at byte (rt * ceil(cb / 4) + ct) * 512).  Inside a
 * tile, S[rt*128 + 32*i + j][ct*4 + k] (i, k < 4, j < 32) sits at byte
 * 16*j + 4*i + k: each 16-byte line holds rows j, j+32, j+64, j+96.
 */
int64_t oracle_swizzled_scale_bytes(int64_t rows, int64_t cb)
{
    int64_t rt = (rows + 127) / 128, ct = (cb + 3) / 4;
    return rt * ct * 512;
}

void oracle_swizzle_scales(const uint8_t *s, int64_t rows, int64_t cb, uint8_t *out)
{
    int64_t ctiles = (cb + 3) / 4;
    int64_t total = oracle_swizzled_scale_bytes(rows, cb);
    for (int64_t i = 0; i < total; i++)
        out[i] = 0;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t c = 0; c < cb; c++) {
            int64_t tile = (r / 128) * ctiles + c / 4;
            int64_t inner = 16 * (r % 32) + 4 * ((r % 128) / 32) + (c % 4);
            out[tile * 512 + inner] = s[r * cb + c];
        }
    }
}
