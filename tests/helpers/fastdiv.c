/*
 * Proof by enumeration that the kernels' three-operation quotient
 *
 *     r  = RN(1/d)                       (one correctly rounded division)
 *     q0 = RN(y * r)                     (fma(y, r, +0))
 *     e  = RN(y - d * q0)                (fma(-q0, d, y); exact in range)
 *     q1 = RN(q0 + e * r)                (fma(e, r, q0))
 *
 * (Markstein's correction step: P. Markstein, "Computation of elementary
 * functions on the IBM RISC System/6000 processor", IBM J. Res. Dev. 34(1),
 * 1990; also J.-M. Muller et al., Handbook of Floating-Point Arithmetic,
 * section on Newton-Raphson-based division) gives the same E2M1 code and the
 * same E4M3 scale as the correctly rounded quotient RN(y/d), for every input
 * the kernels feed it.
 *
 * Why windows suffice: q1 is within one unit in the last place of RN(y/d), so
 * the two can only round to different codes when y/d lies within a few ulps
 * of a decision boundary.  Rounding is invariant under scaling d and y by the
 * same power of two while nothing over- or underflows, so it is enough to
 * enumerate every binary32 significand of d in [1, 2) and, for each decision
 * value t, every y within `w` ulps of RN(d * t).  Every case is compared bit
 * for bit with C's binary32 division (IEEE round to nearest even).
 *
 * The element quotients use a two-operation form instead (verify_element2,
 * verify_random_codes2 below): exact codes, not exact quotients.
 *
 * Test code: built and run by tests/test_fastdiv_cpu.py.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline float fbits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static inline uint32_t bitsf(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static inline float mk(float y, float d, float r)
{
    float q0 = fmaf(y, r, 0.0f);
    float e = fmaf(-q0, d, y);
    return fmaf(e, r, q0);
}

/*
 * Element quotients, in the kernels' scaled form: z = 4y (the unscaled
 * butterfly output) divided by d4 = 4d with r4 = RN(1/d4).  Decision values:
 * the seven E2M1 midpoints.  d ranges over [1, 2) (all 2^23 significands);
 * returns the number of (d, z) pairs where mk differs from z / d4 and stores
 * one example.
 */
long long verify_element(int w, uint32_t *ex_d, uint32_t *ex_z)
{
    static const float T[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
    long long bad = 0;
    uint32_t bd = 0, bz = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t D = 0; D < (1 << 23); D++) {
        float d = fbits(0x3F800000u | (uint32_t)D);      /* [1, 2) */
        float d4 = 4.0f * d;
        float r4 = 1.0f / d4;
        for (int k = 0; k < 7; k++) {
            float c = d4 * T[k];
            uint32_t cb = bitsf(c);
            for (int j = -w; j <= w; j++) {
                float z = fbits(cb + (uint32_t)j);
                float want = z / d4;
                float got = mk(z, d4, r4);
                if (bitsf(want) != bitsf(got)) {
                    bad++;
#pragma omp critical
                    { bd = bitsf(d4); bz = bitsf(z); }
                }
            }
        }
    }
    *ex_d = bd;
    *ex_z = bz;
    return bad;
}

/*
 * Block values v = a6 / g: decision values are the E4M3 midpoints, whose
 * significands are 1 + j/16 for j = 0..15 (odd j: midpoints between normal
 * E4M3 values; even j: midpoints between subnormal ones, 2^-10 included; 464,
 * the boundary of the clamp to 448, is 1.8125 * 2^8).
 */
long long verify_block(int w, uint32_t *ex_g, uint32_t *ex_a)
{
    long long bad = 0;
    uint32_t bg = 0, ba = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t G = 0; G < (1 << 23); G++) {
        float g = fbits(0x3F800000u | (uint32_t)G);
        float rg = 1.0f / g;
        for (int j = 0; j < 16; j++) {
            float c = g * (1.0f + (float)j / 16.0f);
            uint32_t cb = bitsf(c);
            for (int i = -w; i <= w; i++) {
                float a = fbits(cb + (uint32_t)i);
                float want = a / g;
                float got = mk(a, g, rg);
                if (bitsf(want) != bitsf(got)) {
                    bad++;
#pragma omp critical
                    { bg = bitsf(g); ba = bitsf(a); }
                }
            }
        }
    }
    *ex_g = bg;
    *ex_a = ba;
    return bad;
}

/* a / c with the constant r = RN(1/c), every positive binary32 in [lo, hi]
   (c = 6: the block value of an unrotated block; c = 24: of a rotated one,
   whose butterfly output z = 4y enters unscaled, z / 24 = y / 6 exactly) */
long long verify_div_const(float c, uint32_t lo, uint32_t hi, uint32_t *ex)
{
    const float r = 1.0f / c;
    long long bad = 0;
    uint32_t b = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t u = lo; u <= (int64_t)hi; u++) {
        float a = fbits((uint32_t)u);
        if (bitsf(a / c) != bitsf(mk(a, c, r))) {
            bad++;
#pragma omp critical
            b = (uint32_t)u;
        }
    }
    *ex = b;
    return bad;
}

/*
 * The global scale (a / 6) / 448 as two corrected products with the
 * constants RN(1/6) and RN(1/448), against the two binary32 divisions, for
 * every binary32 a in [lo, hi] (the kernels' fast path: [2^-38, 2^15)).
 */
long long verify_global_scale(uint32_t lo, uint32_t hi, uint32_t *ex)
{
    const float r6 = 1.0f / 6.0f, r448 = 1.0f / 448.0f;
    long long bad = 0;
    uint32_t b = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t u = lo; u <= (int64_t)hi; u++) {
        float a = fbits((uint32_t)u);
        float want = (a / 6.0f) / 448.0f;
        float got = mk(mk(a, 6.0f, r6), 448.0f, r448);
        if (bitsf(want) != bitsf(got)) {
            bad++;
#pragma omp critical
            b = (uint32_t)u;
        }
    }
    *ex = b;
    return bad;
}

/*
 * Random pairs over the whole range the kernels allow (d in [2^-62, 2^15],
 * z = 4y a multiple of 2^-133 with |z| <= 6.5 d or arbitrary below d):
 * the E2M1 code from q1 (sign bit for a quotient below zero, -0 and +0 both
 * code 0) must equal the code of RN(z/d).  `n` pairs from a SplitMix64 stream.
 */
static inline uint64_t sm64(uint64_t *s)
{
    uint64_t z = (*s += 0x9e3779b97f4a7c15ULL);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

static int code_of(float v)
{
    float a = fabsf(v);
    int m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
            (a >= 3.5f) + (a > 5.0f);
    return m + (v < 0.0f ? 8 : 0);
}

long long verify_random_codes(int64_t n, uint64_t seed, double *max_ulp_seen)
{
    long long bad = 0;
    double mx = 0.0;
#pragma omp parallel reduction(+ : bad) reduction(max : mx)
    {
        uint64_t s = seed * 0x632be59bd9b4e019ULL + 1;
#ifdef _OPENMP
        extern int omp_get_thread_num(void);
        s += (uint64_t)omp_get_thread_num() * 0x9e3779b97f4a7c15ULL * 7;
#endif
#pragma omp for schedule(static)
        for (int64_t i = 0; i < n; i++) {
            uint64_t a = sm64(&s), b = sm64(&s);
            /* d = 4 * (scale) in [2^-60, 2^15] */
            int de = -60 + (int)(a % 76);
            float d4 = ldexpf(1.0f + (float)((a >> 8) & 0x7FFFFF) / 8388608.0f, de);
            float r4 = 1.0f / d4;
            /* z: mostly |z/d4| in [0, 6.5], sometimes tiny; multiple of 2^-133 */
            float z;
            int kind = (int)(b & 7);
            if (kind < 6) {
                z = (float)((double)d4 * 6.5 * ((double)(b >> 11) * 0x1.0p-53));
            } else {
                int ze = -133 + (int)((b >> 3) % 140);
                z = ldexpf((float)((b >> 11) & 0xFFFF) / 65536.0f + 1.0f, ze);
            }
            if ((b >> 63) & 1)
                z = -z;
            if (fabsf(z) < 0x1p-133f)
                z = 0.0f;
            float want = z / d4;
            float got = mk(z, d4, r4);
            if (code_of(want) != code_of(got + 0.0f) || (got == 0.0f && signbit(got)))
                bad++;
            if (bitsf(want) != bitsf(got)) {
                double u = fabs((double)want - (double)got) /
                           (double)(nextafterf(fabsf(want), INFINITY) - fabsf(want));
                if (u > mx)
                    mx = u;
            }
        }
    }
    *max_ulp_seen = mx;
    return bad;
}

/*
 * Two-operation element quotient.  Once per divisor D (per scale byte, in a
 * table): rh = RN(1/D); e = RN(1 - rh D), exact as one fma; rl = RN(e / D),
 * a correctly rounded division.  Per element: p = RN(z rl + 0) (fma with +0,
 * so that a zero z gives +0), q = RN(z rh + p) (fma).
 *
 * rh + rl equals 1/D within about 2^-47 relative, and p adds an error below
 * 2^-48 of the quotient, so q = RN(Q (1 + eps)) with |eps| < 2^-46 and
 * Q = z / D exactly: q is RN(Q) or an adjacent binary32, and its E2M1 code can
 * differ from that of RN(Q) only where Q lies within about two ulps of one of
 * the seven midpoints.  verify_element2 enumerates exactly those inputs, for
 * every significand of D, and compares codes (the quotient bits may differ
 * by an ulp away from a midpoint; the code never does).  Rounding is
 * invariant under a common power-of-two scaling of z and D while nothing
 * under- or overflows, which holds for the tables the kernels build (D in
 * [2^-57, 2^15): rl is a normal number and z rl stays far from the underflow
 * threshold wherever Q is near a midpoint; a nonzero z, a multiple of
 * 2^-133, gives |Q| >= 2^-148, so q is never a zero of the wrong sign).
 *
 * The tail must be the correctly rounded e / D: with RN(e rh) instead,
 * D = 8 (1 - 2^-24) and z = 2 give rh + rl = (1 + 2^-24) / 8 exactly, so that
 * Q = 0.25 (1 + 2^-24 + 2^-48 + ...), just above the rounding boundary
 * between 0.25 and its successor, is approximated by the boundary itself and
 * rounds (to even) to 0.25: code 0 instead of 1.
 */
static inline void recip2(float d, float *rh, float *rl)
{
    float r = 1.0f / d;
    float e = fmaf(-r, d, 1.0f);
    *rh = r;
    *rl = e / d;
}

static inline float q2(float z, float rh, float rl)
{
    float p = fmaf(z, rl, 0.0f);
    return fmaf(z, rh, p);
}

long long verify_element2(int w, uint32_t *ex_d, uint32_t *ex_z)
{
    static const float T[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
    long long bad = 0;
    uint32_t bd = 0, bz = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t D = 0; D < (1 << 23); D++) {
        float d4 = 4.0f * fbits(0x3F800000u | (uint32_t)D);
        float rh, rl;
        recip2(d4, &rh, &rl);
        for (int k = 0; k < 7; k++) {
            uint32_t cb = bitsf(d4 * T[k]);
            for (int j = -w; j <= w; j++) {
                float z = fbits(cb + (uint32_t)j);
                for (int sg = 0; sg < 2; sg++) {
                    float zz = sg ? -z : z;
                    float got = q2(zz, rh, rl);
                    if (code_of(zz / d4) != code_of(got)) {
                        bad++;
#pragma omp critical
                        { bd = bitsf(d4); bz = bitsf(zz); }
                    }
                }
            }
        }
    }
    *ex_d = bd;
    *ex_z = bz;
    return bad;
}

/*
 * The tail rl = RN(e / D) of the two-word reciprocal by the corrected product
 * instead of a division: e = RN(1 - rh D) (exact as one fma), then
 * mk(e, D, rh).  Compared bit for bit with e / D for every significand of D in
 * every binade from 2^lo_exp to 2^hi_exp (the kernels' tables hold
 * D in [2^-60, 2^16)); returns the number of mismatches and stores one D.
 * Scaling D by 2^k scales rh, rl and every step of mk by 2^-k and leaves e
 * unchanged, so one binade decides all binades in which nothing underflows;
 * enumerating the extreme binades as well checks that.
 */
long long verify_recip_tail(int lo_exp, int hi_exp, uint32_t *ex_d)
{
    long long bad = 0;
    uint32_t bd = 0;
    for (int ex = lo_exp; ex < hi_exp; ex++) {
#pragma omp parallel for schedule(static) reduction(+ : bad)
        for (int64_t D = 0; D < (1 << 23); D++) {
            float d = fbits((uint32_t)(ex + 127) << 23 | (uint32_t)D);
            float rh = 1.0f / d;
            float e = fmaf(-rh, d, 1.0f);
            float want = e / d;
            float got = mk(e, d, rh);
            if (bitsf(want) != bitsf(got)) {
                bad++;
#pragma omp critical
                bd = bitsf(d);
            }
        }
    }
    *ex_d = bd;
    return bad;
}

/* Largest |(rh + rl) D - 1| over every significand of D, in units of 2^-48
   (extended precision; the argument above needs it below 2). */
double max_tail_error(void)
{
    double mx = 0.0;
#pragma omp parallel for schedule(static) reduction(max : mx)
    for (int64_t D = 0; D < (1 << 23); D++) {
        float d = fbits(0x3F800000u | (uint32_t)D);
        float rh, rl;
        recip2(d, &rh, &rl);
        long double err = fabsl(((long double)rh + (long double)rl) * (long double)d - 1.0L);
        double u = (double)(err * 0x1p48L);
        if (u > mx)
            mx = u;
    }
    return mx;
}

/*
 * Random pairs over the whole range the kernels allow, as verify_random_codes
 * but for the two-operation quotient: the code of q (a zero must come out as
 * +0, which the sign rule gives code 0) equals the code of RN(z / D).
 */
long long verify_random_codes2(int64_t n, uint64_t seed)
{
    long long bad = 0;
#pragma omp parallel reduction(+ : bad)
    {
        uint64_t s = seed * 0x632be59bd9b4e019ULL + 1;
#ifdef _OPENMP
        extern int omp_get_thread_num(void);
        s += (uint64_t)omp_get_thread_num() * 0x9e3779b97f4a7c15ULL * 7;
#endif
#pragma omp for schedule(static)
        for (int64_t i = 0; i < n; i++) {
            uint64_t a = sm64(&s), b = sm64(&s);
            int de = -60 + (int)(a % 76);   /* D in [2^-60, 2^16) */
            float d4 = ldexpf(1.0f + (float)((a >> 8) & 0x7FFFFF) / 8388608.0f, de);
            float rh, rl;
            recip2(d4, &rh, &rl);
            float z;
            int kind = (int)(b & 7);
            if (kind < 6) {
                z = (float)((double)d4 * 6.5 * ((double)(b >> 11) * 0x1.0p-53));
            } else {
                int ze = -133 + (int)((b >> 3) % 140);
                z = ldexpf((float)((b >> 11) & 0xFFFF) / 65536.0f + 1.0f, ze);
            }
            if ((b >> 63) & 1)
                z = -z;
            if (fabsf(z) < 0x1p-133f)
                z = ((b >> 62) & 1) ? -0.0f : 0.0f;
            float got = q2(z, rh, rl);
            if (code_of(z / d4) != code_of(got) || (got == 0.0f && signbit(got)))
                bad++;
        }
    }
    return bad;
}
