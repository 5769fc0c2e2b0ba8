// Device building blocks of the rotate+quantize kernels (gfx950).
//
// Method: page "A Fused Hadamard + NVFP4 Quantization Kernel in Triton"
// (kanthi.in), sections 1-3.  Every helper below computes exactly the binary32
// operation of that definition, or a sequence proven to give the same bits
// where it is used (see the notes on div_corrected and on the conversions).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace nvfp4rq {

// ---------------------------------------------------------------- widening

// bf16 is the top half of a binary32, so widening is a shift or a mask: exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 16 bytes = 8 consecutive bf16 values, element order preserved.
__device__ __forceinline__ void widen8(uint4 a, float z[8]) {
  z[0] = bf16_lo(a.x);
  z[1] = bf16_hi(a.x);
  z[2] = bf16_lo(a.y);
  z[3] = bf16_hi(a.y);
  z[4] = bf16_lo(a.z);
  z[5] = bf16_hi(a.z);
  z[6] = bf16_lo(a.w);
  z[7] = bf16_hi(a.w);
}

// ---------------------------------------------------------------- rotation

// H16 = S16 / 4 with S16 the Sylvester matrix built by four Kronecker
// doublings [[H, H], [H, -H]] (section 1; section 2, hadamard16).  S16 z is
// the butterfly with strides 1, 2, 4, 8, each stage replacing a pair (a, b) by
// (a + b, a - b).  These helpers run the stages in that order on values held
// in registers; the final multiply by 0.25 is applied by the caller (or folded
// into an exactly scaled divisor).

// strides 1, 2, 4 on 8 consecutive elements
__device__ __forceinline__ void stages_1_2_4(float z[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & h) == 0) {
        const float a = z[i];
        const float b = z[i + h];
        z[i] = a + b;
        z[i + h] = a - b;
      }
    }
  }
}

// strides 1, 2 on 4 consecutive elements
__device__ __forceinline__ void stages_1_2(float z[4]) {
#pragma unroll
  for (int h = 1; h < 4; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if ((i & h) == 0) {
        const float a = z[i];
        const float b = z[i + h];
        z[i] = a + b;
        z[i + h] = a - b;
      }
    }
  }
}

// stride-8 stage for a block whose elements 0..7 are in lo and 8..15 in hi
__device__ __forceinline__ void stage_8(float lo[8], float hi[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = lo[i];
    const float b = hi[i];
    lo[i] = a + b;
    hi[i] = a - b;
  }
}

// Lane exchange with the neighbouring lane (quad_perm [1,0,3,2]); the
// compiler folds it into the consuming VALU instruction as a DPP operand.
__device__ __forceinline__ float swap_lane1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}

// Lane exchange within a quad: quad_perm [2,3,0,1] (lane ^ 2).
__device__ __forceinline__ float swap_lane2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// Strides 4 and 8 for a block spread over the four lanes of a quad, lane t of
// the quad holding elements 4t..4t+3 (strides 1 and 2 already applied in
// lane).  Stride 4 pairs lanes t and t^1, stride 8 lanes t and t^2.  The lane
// that holds the pair's first element a keeps a + b; its partner, holding b,
// forms a - b as a + (-b), which is the same binary32 operation.  Every lane
// of the quad must execute this (the exchange reads the partner's register).
__device__ __forceinline__ void quad_stages_4_8(float z[4], uint32_t lane) {
  const uint32_t s1 = (lane & 1u) << 31, s2 = (lane & 2u) << 30;
#pragma unroll
  for (int i = 0; i < 4; ++i) z[i] = swap_lane1(z[i]) + __uint_as_float(__float_as_uint(z[i]) ^ s1);
#pragma unroll
  for (int i = 0; i < 4; ++i) z[i] = swap_lane2(z[i]) + __uint_as_float(__float_as_uint(z[i]) ^ s2);
}

// ---------------------------------------------------------------- division

// RN(1/6) and RN(1/24) = RN(1/6) / 4 as binary32.
constexpr float kRecip6 = 0.16666667163372040f;
constexpr float kRecip24 = 0.041666667908430100f;

// Correctly rounded y / d given r = RN(1/d): Markstein's correction step,
// q0 = RN(y r), e = y - d q0 (exact), q1 = RN(q0 + e r).  q0 adds +0 so that a
// zero y gives +0 whatever the signs of y, d and r.  Enumerated on the CPU
// (tests/helpers/fastdiv.c): equal to IEEE division at every input near an
// E4M3 decision boundary for every divisor significand, and for the divides
// by 6 and by 24 at every input >= 2^-124 and >= 2^-122.
__device__ __forceinline__ float div_corrected(float y, float d, float r) {
  const float q0 = __builtin_fmaf(y, r, 0.0f);
  const float e = __builtin_fmaf(-q0, d, y);
  return __builtin_fmaf(e, r, q0);
}

// Two-word reciprocal of D: rh = RN(1/D) and rl = RN(e / D) with the
// residual e = 1 - rh D, exact as one fused multiply-add.  rh + rl is 1/D
// within 2^-47 relative.  rh is a correctly rounded division; rl comes from
// the corrected product div_corrected(e, D, rh), which equals the correctly
// rounded e / D for every binary32 D in [2^-60, 2^16), the range of the
// kernels' tables (enumerated on the CPU, tests/helpers/fastdiv.c).
__device__ __forceinline__ float2 recip2_corrected(float d) {
  const float rh = 1.0f / d;
  return make_float2(rh, div_corrected(__builtin_fmaf(-rh, d, 1.0f), d, rh));
}

// z / D from its two-word reciprocal (rh, rl): p = RN(z rl + 0),
// q = RN(z rh + p).  q is RN(z/D (1 + eps)) with |eps| < 2^-46, so it is the
// correctly rounded quotient or an adjacent binary32; its E2M1 code equals
// that of the correctly rounded quotient for every input of the kernels'
// fast path (exhaustive over the inputs near every E2M1 decision boundary,
// for every divisor significand, tests/helpers/fastdiv.c).  A zero z gives
// +0 (the +0 of p absorbs a -0 product).
__device__ __forceinline__ float quot2(float z, float rh, float rl) {
  const float p = __builtin_fmaf(z, rl, 0.0f);
  return __builtin_fmaf(z, rh, p);
}

// ---------------------------------------------------------------- conversions

// E4M3FN byte of min(round-to-nearest-even(v), 448), v >= 0.  The gfx950
// conversion instruction (v_cvt_pk_fp8_f32) rounds to nearest even onto the
// OCP E4M3FN grid, subnormals included; an exhaustive sweep of every binary32
// in [0, 448] matches the definition (tests/test_instructions_gpu.py).  Above
// 464 it would give NaN, hence the clamp first: min(v, 448) rounds to the
// same byte as min(round(v), 448) (section 2, _round_e4m3; section 3).
// e4m3_byte_lo leaves bits 8..31 of the result unspecified (the instruction
// writes only the low half; the other bits are those of an unrelated
// register), for callers that use the low byte alone.
__device__ __forceinline__ uint32_t e4m3_byte_lo(float v) {
  const float c = __builtin_fminf(v, 448.0f);
  return static_cast<uint32_t>(
      __builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, static_cast<int>(__float_as_uint(v)), false));
}
__device__ __forceinline__ uint32_t e4m3_byte(float v) { return e4m3_byte_lo(v) & 0xFFu; }

// Value of an E4M3FN byte (exact).
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(b), 0);
}

// Eight quotients -> one dword of E2M1 codes, element 2k in the low nibble of
// byte k (section 2: two codes per byte, even element low).  The gfx950
// conversion (v_cvt_scalef32_pk_fp4_f32 with scale 1.0) rounds to the nearest
// grid magnitude with ties to the even code, saturates beyond 6, and sets the
// sign bit from the IEEE sign: an exhaustive sweep of every non-NaN binary32
// matches the page's midpoint compares except at -0.0 (hardware 8, the page
// 0 since -0.0 < 0 is false).  Callers therefore never pass -0.0: the
// corrected quotient returns +0 for any zero input, and the exact path adds
// +0.0 (which turns -0.0 into +0.0 and leaves every other value unchanged).
// The four conversions write one byte each, so the destination's initial
// bits never reach the result; they are taken from q[0], whose register is
// free after the first conversion (no register has to be zeroed first).
__device__ __forceinline__ uint32_t e2m1_pack8(const float q[8]) {
  uint32_t w = __float_as_uint(q[0]);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[0], q[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[2], q[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[4], q[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[6], q[7], 1.0f, 3);
  return w;
}

// Signed grid values of the two E2M1 codes in byte BYTE of w, element 2k in
// the low nibble (section 1 table; section 2, dequantize's GRID):
// +-{0, .5, 1, 1.5, 2, 3, 4, 6}[c & 7], code 8 giving -0.0 like the page's
// sign flip of a zero magnitude.  The gfx950 conversion
// v_cvt_scalef32_pk_f32_fp4 with scale 1.0 returns both values exactly; a
// check of all 256 bytes at each of the four byte positions matches the table
// bit for bit (tests/test_instructions_gpu.py).  Only the exponent of the
// scale operand enters the instruction, so the block scale is applied by an
// ordinary binary32 multiply afterwards.
template <int BYTE>
__device__ __forceinline__ float2 e2m1_pair(uint32_t w) {
  const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, BYTE);
  return make_float2(v[0], v[1]);
}

// ---------------------------------------------------------------- scales

// Global scale (section 1 table; section 2, quantize): (amax / 6) / 448 as two
// binary32 divisions, 1.0 when that is zero.
__device__ __forceinline__ float global_scale(float amax) {
  const float g = (amax / 6.0f) / 448.0f;
  return g == 0.0f ? 1.0f : g;
}

// The same two divisions as corrected products, for amax in [2^-38, 2^15)
// (the kernels' fast path): a / 6 gives the correctly rounded quotient for
// every a >= 2^-124, and y / 448 for every y in [2^-41, 2^13), which holds
// every y = RN(amax / 6) here (both enumerated over every binary32 in range,
// tests/helpers/fastdiv.c); the result is never zero there.
constexpr float kRecip448 = 1.0f / 448.0f;
__device__ __forceinline__ float global_scale_corrected(float amax) {
  return div_corrected(div_corrected(amax, 6.0f, kRecip6), 448.0f, kRecip448);
}

}  // namespace nvfp4rq
