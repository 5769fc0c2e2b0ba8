/*
 * Seeded synthetic activation tensors for the tests and the benchmark.
 *
 * This module only draws numbers.  It holds none of the quantizer's
 * arithmetic: no amax, no scale, no rounding to E4M3 or E2M1.  Both the CPU
 * oracle and the HIP library receive the bytes it writes, and nothing else
 * flows between them.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014) used as a counter-based generator: draw i of
 * stream k is mix64(key_k + (i + 1) * 0x9e3779b97f4a7c15), where key_k is a
 * hash of (seed, k).  Every value is therefore a pure function of
 * (seed, stream, index), independent of the thread count and of which slice of
 * a tensor is generated.  Normals use the Box-Muller transform on two 53-bit
 * uniforms; every value is computed in fp64 and rounded once, to bf16 (round
 * to nearest even, computed directly from the double) or to binary32.
 *
 * Workload recipes (shapes and value structure follow the pages' test tensors
 * and the activation shapes they discuss):
 *   gauss_outliers  N(0,1) with a few whole columns scaled up - the
 *                   outlier-channel tensor of "A Fused Hadamard + NVFP4
 *                   Quantization Kernel in Triton", section 3;
 *   t3_lognormal    Student-t (3 d.o.f.) times a per-column log-normal gain -
 *                   the heavy-tailed case of the same page, section 5;
 *   silu_ties       SiLU(a) * b, the shape of an MLP intermediate, with planted
 *                   blocks whose scaled values sit exactly on the E2M1
 *                   midpoints and an anchor block that fixes a power-of-two
 *                   global scale;
 *   kv_heads        fp32 [tokens, heads, 128] with a per-head scale, planted
 *                   all-zero, all-negative-zero and dominant (saturating)
 *                   blocks - the KV-cache layout of the page "NVFP4
 *                   Quantization" (atlas-docs), section "NVFP4 KV cache".
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

#define GOLDEN 0x9e3779b97f4a7c15ULL

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream)
{
    return mix64(mix64(seed + GOLDEN) ^ mix64(stream * 0xd1b54a32d192ed03ULL + 1));
}

static inline uint64_t draw(uint64_t key, uint64_t i)
{
    return mix64(key + (i + 1) * GOLDEN);
}

/* uniform in [0, 1) with 53 random bits */
static inline double u01(uint64_t key, uint64_t i)
{
    return (double)(draw(key, i) >> 11) * 0x1.0p-53;
}

/* uniform in (0, 1] */
static inline double u01_open0(uint64_t key, uint64_t i)
{
    return (double)((draw(key, i) >> 11) + 1) * 0x1.0p-53;
}

/* standard normal number i of a stream (Box-Muller, cosine branch) */
static inline double normal(uint64_t key, uint64_t i)
{
    double u1 = u01_open0(key, 2 * i);
    double u2 = u01(key, 2 * i + 1);
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

/* fp64 -> bf16 bits, round to nearest, ties to even, in one step */
static uint16_t f64_to_bf16(double d)
{
    uint16_t sign = signbit(d) ? 0x8000 : 0;
    double a = fabs(d);
    if (a == 0.0)
        return sign;
    if (isinf(a) || a >= 0x1.ffp127)        /* beyond the largest finite bf16: saturate */
        return (uint16_t)(sign | 0x7F7F);
    int e;
    (void)frexp(a, &e);                      /* a in [2^(e-1), 2^e) */
    int q = e - 1 - 7;                       /* quantum of an 8-bit significand */
    if (q < -133)
        q = -133;                            /* bf16 subnormal quantum */
    double k = ldexp(a, -q);                 /* exact scaling */
    double kf = floor(k);
    double fr = k - kf;
    if (fr > 0.5 || (fr == 0.5 && fmod(kf, 2.0) == 1.0))
        kf += 1.0;
    float f = (float)ldexp(kf, q);           /* <= 9 significant bits: exact */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

static float f64_to_f32(double d)
{
    return (float)d;                         /* one IEEE rounding, nearest-even */
}

/* ------------------------------------------------------------------ */
/* exported primitives                                                  */
/* ------------------------------------------------------------------ */

void synth_normal_f64(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, double *out)
{
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = normal(key, start + (uint64_t)i);
}

void synth_uniform_f64(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, double *out)
{
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = u01(key, start + (uint64_t)i);
}

void synth_round_bf16(const double *in, int64_t n, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = f64_to_bf16(in[i]);
}

/* n normals times `scale`, rounded to bf16 or binary32 */
void synth_normal_bf16(uint64_t seed, uint64_t stream, int64_t n, double scale, uint16_t *out)
{
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = f64_to_bf16(scale * normal(key, (uint64_t)i));
}

void synth_normal_f32(uint64_t seed, uint64_t stream, int64_t n, double scale, float *out)
{
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = f64_to_f32(scale * normal(key, (uint64_t)i));
}

/* ------------------------------------------------------------------ */
/* column choice                                                        */
/* ------------------------------------------------------------------ */

/* k distinct columns out of `cols`, by a partial Fisher-Yates shuffle */
static int pick_columns(uint64_t key, int64_t cols, int64_t k, int64_t *picked)
{
    int64_t *perm = (int64_t *)malloc((size_t)cols * sizeof(int64_t));
    if (!perm)
        return -1;
    for (int64_t c = 0; c < cols; c++)
        perm[c] = c;
    for (int64_t i = 0; i < k; i++) {
        int64_t j = i + (int64_t)(draw(key, (uint64_t)i) % (uint64_t)(cols - i));
        int64_t t = perm[i];
        perm[i] = perm[j];
        perm[j] = t;
        picked[i] = perm[i];
    }
    free(perm);
    return 0;
}

/* ------------------------------------------------------------------ */
/* recipes                                                              */
/* ------------------------------------------------------------------ */

/*
 * N(0,1) bf16 [rows, cols]; n_out distinct columns (chosen by the generator)
 * are multiplied by a per-column factor drawn from U(lo, hi) (lo == hi gives a
 * fixed factor).  The chosen columns are written to picked_out when not NULL.
 */
int synth_gauss_outliers(uint64_t seed, int64_t rows, int64_t cols, int64_t n_out,
                         double lo, double hi, uint16_t *out, int64_t *picked_out)
{
    if (n_out < 0 || n_out > cols)
        return -1;
    uint64_t kval = stream_key(seed, 1);
    uint64_t kcol = stream_key(seed, 2);
    uint64_t kfac = stream_key(seed, 3);
    double *factor = (double *)malloc((size_t)(cols > 0 ? cols : 1) * sizeof(double));
    int64_t *picked = (int64_t *)malloc((size_t)(n_out > 0 ? n_out : 1) * sizeof(int64_t));
    if (!factor || !picked) {
        free(factor);
        free(picked);
        return -1;
    }
    for (int64_t c = 0; c < cols; c++)
        factor[c] = 1.0;
    if (n_out > 0 && pick_columns(kcol, cols, n_out, picked) != 0) {
        free(factor);
        free(picked);
        return -1;
    }
    for (int64_t i = 0; i < n_out; i++) {
        factor[picked[i]] = lo + (hi - lo) * u01(kfac, (uint64_t)i);
        if (picked_out)
            picked_out[i] = picked[i];
    }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++) {
            uint64_t i = (uint64_t)(r * cols + c);
            out[r * cols + c] = f64_to_bf16(normal(kval, i) * factor[c]);
        }
    free(factor);
    free(picked);
    return 0;
}

/*
 * Student-t with 3 degrees of freedom, built as Z / sqrt((Z1^2+Z2^2+Z3^2)/3),
 * times a per-column gain exp(n_c) with n_c ~ N(0,1) (a log-normal(0,1) gain).
 */
int synth_t3_lognormal(uint64_t seed, int64_t rows, int64_t cols, uint16_t *out)
{
    uint64_t kz = stream_key(seed, 11);
    uint64_t k1 = stream_key(seed, 12);
    uint64_t k2 = stream_key(seed, 13);
    uint64_t k3 = stream_key(seed, 14);
    uint64_t kg = stream_key(seed, 15);
    double *gain = (double *)malloc((size_t)(cols > 0 ? cols : 1) * sizeof(double));
    if (!gain)
        return -1;
    for (int64_t c = 0; c < cols; c++)
        gain[c] = exp(normal(kg, (uint64_t)c));
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++) {
            uint64_t i = (uint64_t)(r * cols + c);
            double z = normal(kz, i);
            double a = normal(k1, i), b = normal(k2, i), d = normal(k3, i);
            double t = z / sqrt((a * a + b * b + d * d) / 3.0);
            out[r * cols + c] = f64_to_bf16(t * gain[c]);
        }
    free(gain);
    return 0;
}

/* Sylvester sign (-1)^popcount(i & j) */
static inline int syl_sign(int i, int j)
{
    return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1 : 1;
}

/* the E2M1 midpoints, scaled so that they are the values a tie block holds */
static const double TIE_VALUES[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};

/*
 * SiLU(a) * b with a, b ~ N(0,1), bf16 [rows, cols] (cols % 16 == 0), plus:
 *  - one anchor block whose largest |value| after the block rotation (when
 *    `rotate`) or as stored (when not) is exactly 168 = 2688 / 16, larger than
 *    every natural value, so that 168 / 6 / 448 = 1/16 exactly;
 *  - about one block in 1024 holding a "tie block": its target values t_j are
 *    drawn from +-{0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5} with one entry +-6.
 *    With the anchor's scale 1/16, a block whose largest magnitude is 6 gets
 *    the scale 16 and the divisor 16/16 = 1, so every t_j is an exact E2M1
 *    midpoint.  When `rotate`, the block stores H16 * t (the inverse of the
 *    orthonormal symmetric block rotation), computed exactly with the Sylvester
 *    signs: every entry is a multiple of 1/16 below 21, and a draw is kept only
 *    when all 16 entries are exact in bf16 (otherwise the next draw is tried),
 *    so the rotation of the stored block gives t back without rounding.
 * Writes the anchor block index to *anchor_block and the number of tie blocks
 * to *n_tie (either may be NULL); tie_flags (one byte per block, may be NULL)
 * marks the tie blocks.
 */
int synth_silu_ties(uint64_t seed, int64_t rows, int64_t cols, int rotate, uint16_t *out,
                    int64_t *anchor_block, int64_t *n_tie, uint8_t *tie_flags)
{
    if (cols % 16 != 0 || rows <= 0 || cols <= 0)
        return -1;
    uint64_t ka = stream_key(seed, 21);
    uint64_t kb = stream_key(seed, 22);
    uint64_t kt = stream_key(seed, 23);
    uint64_t kv = stream_key(seed, 24);
    uint64_t kanc = stream_key(seed, 25);
    int64_t nb = rows * (cols / 16);
    int64_t anchor = (int64_t)(draw(kanc, 0) % (uint64_t)nb);
    int64_t ties = 0;
#pragma omp parallel for schedule(static) reduction(+ : ties)
    for (int64_t blk = 0; blk < nb; blk++) {
        uint16_t *o = out + blk * 16;
        int is_tie = (blk != anchor) && (draw(kt, (uint64_t)blk) >> 54) == 0; /* 1/1024 */
        if (tie_flags)
            tie_flags[blk] = (uint8_t)is_tie;
        if (blk == anchor) {
            if (rotate) {
                for (int i = 0; i < 16; i++)
                    o[i] = f64_to_bf16(42.0);    /* rotates to (168, 0, ..., 0) */
            } else {
                for (int i = 0; i < 16; i++) {
                    uint64_t e = (uint64_t)(blk * 16 + i);
                    double a = normal(ka, e);
                    o[i] = f64_to_bf16(a / (1.0 + exp(-a)) * normal(kb, e));
                }
                o[(int)(draw(kanc, 1) % 16)] = f64_to_bf16(168.0);
            }
            continue;
        }
        if (!is_tie) {
            for (int i = 0; i < 16; i++) {
                uint64_t e = (uint64_t)(blk * 16 + i);
                double a = normal(ka, e);
                o[i] = f64_to_bf16(a / (1.0 + exp(-a)) * normal(kb, e));
            }
            continue;
        }
        ties++;
        for (uint64_t attempt = 0;; attempt++) {
            uint64_t base = ((uint64_t)blk * 64 + attempt) * 32;
            double t[16];
            for (int j = 0; j < 16; j++) {
                uint64_t r = draw(kv, base + (uint64_t)j);
                double mag = TIE_VALUES[r % 7];
                t[j] = ((r >> 32) & 1) ? -mag : mag;
            }
            uint64_t r6 = draw(kv, base + 16);
            t[r6 % 16] = ((r6 >> 32) & 1) ? -6.0 : 6.0;
            if (!rotate) {
                for (int i = 0; i < 16; i++)
                    o[i] = f64_to_bf16(t[i]);
                break;
            }
            int ok = 1;
            uint16_t cand[16];
            for (int i = 0; i < 16 && ok; i++) {
                double acc = 0.0;
                for (int j = 0; j < 16; j++)
                    acc += syl_sign(i, j) * t[j];
                double xi = acc / 4.0;               /* exact: a multiple of 1/16 */
                cand[i] = f64_to_bf16(xi);
                uint32_t u = (uint32_t)cand[i] << 16;
                float back;
                memcpy(&back, &u, sizeof back);
                if ((double)back != xi)
                    ok = 0;
            }
            if (ok || attempt >= 63) {
                /* 64 failed draws never happen in practice; fall back to the
                   unrotated pattern, which is then simply a non-tie block */
                for (int i = 0; i < 16; i++)
                    o[i] = ok ? cand[i] : f64_to_bf16(t[i] / 64.0);
                break;
            }
        }
    }
    if (anchor_block)
        *anchor_block = anchor;
    if (n_tie)
        *n_tie = ties;
    return 0;
}

/*
 * KV-cache shaped fp32 tensor [tokens, heads * dim] (dim % 16 == 0):
 * N(0,1) times a per-head factor sigma_h ~ U(0.1, 10).  Planted blocks,
 * chosen per block by the generator:
 *  - about 1 in 1024 all +0.0;
 *  - about 1 in 65536 all -0.0;
 *  - about 1 in 4096 copies of one "dominant" block of N(0,1) * 200 values,
 *    far above every natural value, so every copy holds the tensor's largest
 *    magnitude (with or without the rotation) and gets the largest block scale.
 * block_kind (one byte per block, may be NULL): 0 natural, 1 zero,
 * 2 negative zero, 3 dominant copy.
 */
int synth_kv_heads(uint64_t seed, int64_t tokens, int64_t heads, int64_t dim, float *out,
                   uint8_t *block_kind)
{
    if (dim % 16 != 0 || tokens <= 0 || heads <= 0)
        return -1;
    int64_t cols = heads * dim;
    uint64_t kx = stream_key(seed, 31);
    uint64_t kh = stream_key(seed, 32);
    uint64_t kk = stream_key(seed, 33);
    uint64_t kd = stream_key(seed, 34);
    double *sigma = (double *)malloc((size_t)heads * sizeof(double));
    if (!sigma)
        return -1;
    for (int64_t h = 0; h < heads; h++)
        sigma[h] = 0.1 + 9.9 * u01(kh, (uint64_t)h);
    float dom[16];
    for (int i = 0; i < 16; i++)
        dom[i] = f64_to_f32(200.0 * normal(kd, (uint64_t)i));
    int64_t nb = tokens * (cols / 16);
    int64_t bpr = cols / 16;
#pragma omp parallel for schedule(static)
    for (int64_t blk = 0; blk < nb; blk++) {
        float *o = out + blk * 16;
        uint64_t r = draw(kk, (uint64_t)blk) >> 48;  /* 16 uniform bits */
        int kind = 0;
        if (r == 0)
            kind = 2;
        else if (r < 16)
            kind = 3;
        else if (r < 80)
            kind = 1;
        if (block_kind)
            block_kind[blk] = (uint8_t)kind;
        if (kind == 1 || kind == 2) {
            for (int i = 0; i < 16; i++)
                o[i] = (kind == 2) ? -0.0f : 0.0f;
            continue;
        }
        if (kind == 3) {
            for (int i = 0; i < 16; i++)
                o[i] = dom[i];
            continue;
        }
        int64_t c0 = (blk % bpr) * 16;
        double sg = sigma[c0 / dim];
        for (int i = 0; i < 16; i++)
            o[i] = f64_to_f32(sg * normal(kx, (uint64_t)(blk * 16 + i)));
    }
    free(sigma);
    return 0;
}
