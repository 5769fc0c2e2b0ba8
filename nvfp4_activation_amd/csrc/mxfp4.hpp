// MXFP4 variant: 32-element blocks with power-of-two (E8M0) scales, one pass.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "nvfp4rq_device.hpp"
#include "common.hpp"

namespace nvfp4rq {
namespace {  // one translation unit (nvfp4rq.hip): internal linkage


// MXFP4 (the contrast format of section 1 of the page: 32-element blocks,
// power-of-two E8M0 scales; the page "Hopper kernel for MXFP4" stores a scale
// as a biased exponent byte, value 2^(byte - 127)).  There is no global scale,
// so this is a single pass: each lane rotates (each 16-element half with H16),
// scales and encodes one 32-element block per iteration.  Readings: the scale
// is the smallest power of two at or above fl(block_amax / 6), exponent
// clamped to [-127, 127], 0 for an all-zero block; v = fl(y / scale), which
// is the exact product y * 2^-e rounded once; then the E2M1 rule of the NVFP4
// path (+0.0 turns an underflowed -0.0 into +0.0: code 0, not 8).
template <typename T, bool ROTATE>
__global__ __launch_bounds__(kThreads) void mx_quant_kernel(const T* __restrict__ x, int64_t nb32,
                                                            uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ s) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; b < nb32; b += stride) {
    float v[4][8];     // halves: (v[0], v[1]) elements 0..15, (v[2], v[3]) 16..31
    load_block(x, 2 * b, v[0], v[1]);
    load_block(x, 2 * b + 1, v[2], v[3]);
    if (ROTATE) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        stages_1_2_4(v[2 * h]);
        stages_1_2_4(v[2 * h + 1]);
        stage_8(v[2 * h], v[2 * h + 1]);
      }
    }
    float az = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) az = __builtin_fmaxf(az, __builtin_fabsf(v[k][i]));
    const float t = (ROTATE ? 0.25f * az : az) / 6.0f;
    int e = -127;
    if (t > 0.0f) {
      int fe;
      const float m = frexpf(t, &fe);          // t = m 2^fe, m in [0.5, 1)
      e = m == 0.5f ? fe - 1 : fe;             // ceil(log2 t)
      e = e < -127 ? -127 : (e > 127 ? 127 : e);
    }
    // bf16: the butterfly output z = 4y is exact and y * 2^-e = z * 2^(-e-2);
    // fp32 values may round when scaled by 0.25, so they are scaled first.
    const bool fold = ROTATE && sizeof(T) == 2;
    const float inv = ldexpf(1.0f, fold ? -e - 2 : -e);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float y = (ROTATE && !fold) ? 0.25f * v[k][i] : v[k][i];
        v[k][i] = y * inv + 0.0f;
      }
    *reinterpret_cast<uint4*>(q + b * 16) =
        make_uint4(e2m1_pack8(v[0]), e2m1_pack8(v[1]), e2m1_pack8(v[2]), e2m1_pack8(v[3]));
    s[b] = static_cast<uint8_t>(e + 127);
  }
}

}  // namespace
}  // namespace nvfp4rq
