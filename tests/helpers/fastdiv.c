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

/* a / 6 with the constant r6 = RN(1/6), every positive binary32 in [lo, hi] */
long long verify_div6(uint32_t lo, uint32_t hi, uint32_t *ex)
{
    const float r6 = 1.0f / 6.0f;
    long long bad = 0;
    uint32_t b = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t u = lo; u <= (int64_t)hi; u++) {
        float a = fbits((uint32_t)u);
        if (bitsf(a / 6.0f) != bitsf(mk(a, 6.0f, r6))) {
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
