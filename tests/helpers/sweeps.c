/*
 * Exhaustive sweeps that pin the oracle's element helpers (test code).
 *
 * Each sweep compares an oracle function with an independent definition
 * written here as a nearest-point search:
 *   - E2M1: nearest of the 8 grid magnitudes {0,.5,1,1.5,2,3,4,6}, an exact tie
 *     going to the even code, sign bit for values below zero (page "A Fused
 *     Hadamard + NVFP4 Quantization Kernel in Triton", sections 1 and 2);
 *   - E4M3: nearest of the 127 non-negative finite E4M3FN values, built here
 *     from the bit-field definition, an exact tie going to the even byte
 *     (even mantissa), everything at or above 448 giving 448 (same page,
 *     sections 1, 2 and 3).
 * Distances below 16 are exact in fp64 except far below the grid, where the
 * nearest point is unambiguous; far above the grid the nearest point is the
 * largest one.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

uint8_t oracle_e2m1_code(float v);
uint8_t oracle_e4m3_byte(float v);
uint8_t oracle_e8m0_byte(float t);

static const double GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

static uint8_t e2m1_nearest(float v)
{
    double a = fabs((double)v);
    int best = 0;
    double bd = INFINITY;
    /* at and above 16 the nearest grid point is plainly the largest one, 6.0;
       below 16 every distance is exact in fp64 */
    if (a >= 16.0)
        return (uint8_t)(7 + (v < 0.0f ? 8 : 0));
    for (int k = 0; k < 8; k++) {
        double d = fabs(a - GRID[k]);
        if (d < bd || (d == bd && (k % 2 == 0))) {
            bd = d;
            best = k;
        }
    }
    return (uint8_t)(best + (v < 0.0f ? 8 : 0));
}

static double E4M3[127];

static void e4m3_table(void)
{
    for (int b = 0; b < 127; b++) {
        int e = b >> 3, m = b & 7;
        E4M3[b] = (e == 0) ? m * ldexp(1.0, -9) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    }
}

static uint8_t e4m3_nearest(float v)
{
    double a = (double)v;
    if (a >= 448.0)
        return 0x7E;
    /* binary search for the first table value >= a, then compare the two
       neighbours (the table is strictly increasing) */
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi) / 2;
        if (E4M3[mid] >= a)
            hi = mid;
        else
            lo = mid + 1;
    }
    if (lo == 0)
        return 0;
    double dl = a - E4M3[lo - 1], dh = E4M3[lo] - a;
    if (dl < dh)
        return (uint8_t)(lo - 1);
    if (dh < dl)
        return (uint8_t)lo;
    return (uint8_t)(((lo - 1) % 2 == 0) ? lo - 1 : lo);
}

/* brute force over all 127 values (slow; used on a subset) */
static uint8_t e4m3_linear(float v)
{
    double a = (double)v;
    if (a >= 448.0)
        return 0x7E;
    int best = 0;
    double bd = INFINITY;
    for (int b = 0; b < 127; b++) {
        double d = fabs(a - E4M3[b]);
        if (d < bd || (d == bd && (b % 2 == 0))) {
            bd = d;
            best = b;
        }
    }
    return (uint8_t)best;
}

static float from_bits(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* every non-NaN binary32 bit pattern; returns the number of mismatches and the
   first mismatching pattern in *first */
long long sweep_e2m1_all(uint32_t *first)
{
    long long bad = 0;
    uint32_t fb = 0xFFFFFFFFu;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t i = 0; i <= 0xFFFFFFFFLL; i++) {
        uint32_t u = (uint32_t)i;
        if ((u & 0x7FFFFFFFu) > 0x7F800000u)
            continue;
        float f = from_bits(u);
        if (oracle_e2m1_code(f) != e2m1_nearest(f)) {
            bad++;
#pragma omp critical
            if (u < fb)
                fb = u;
        }
    }
    *first = fb;
    return bad;
}

/* binary32 patterns lo..hi (non-negative values), nearest search by bisection */
long long sweep_e4m3_range(uint32_t lo, uint32_t hi, uint32_t *first)
{
    e4m3_table();
    long long bad = 0;
    uint32_t fb = 0xFFFFFFFFu;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t i = lo; i <= (int64_t)hi; i++) {
        uint32_t u = (uint32_t)i;
        float f = from_bits(u);
        if (oracle_e4m3_byte(f) != e4m3_nearest(f)) {
            bad++;
#pragma omp critical
            if (u < fb)
                fb = u;
        }
    }
    *first = fb;
    return bad;
}

/* every `stride`-th pattern in lo..hi against the linear search over all 127 */
long long sweep_e4m3_linear(uint32_t lo, uint32_t hi, uint32_t stride, uint32_t *first)
{
    e4m3_table();
    long long bad = 0;
    uint32_t fb = 0xFFFFFFFFu;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t i = lo; i <= (int64_t)hi; i += stride) {
        uint32_t u = (uint32_t)i;
        float f = from_bits(u);
        if (oracle_e4m3_byte(f) != e4m3_linear(f)) {
            bad++;
#pragma omp critical
            if (u < fb)
                fb = u;
        }
    }
    *first = fb;
    return bad;
}

/* E8M0: smallest power of two >= t, by bisection over the 255 exponents
   -127..127 (compared exactly in double), every positive finite binary32. */
long long sweep_e8m0_all(uint32_t *first)
{
    long long bad = 0;
    uint32_t fb = 0xFFFFFFFFu;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t i = 1; i < 0x7F800000LL; i++) {
        uint32_t u = (uint32_t)i;
        float f = from_bits(u);
        double t = (double)f;
        int lo = 0, hi = 254;            /* byte b means 2^(b-127) */
        while (lo < hi) {
            int mid = (lo + hi) / 2;
            if (ldexp(1.0, mid - 127) >= t)
                hi = mid;
            else
                lo = mid + 1;
        }
        if (oracle_e8m0_byte(f) != (uint8_t)lo) {
            bad++;
#pragma omp critical
            if (u < fb)
                fb = u;
        }
    }
    *first = fb;
    return bad;
}
