// Pass 1: the rotated global amax (page "A Fused Hadamard + NVFP4
// Quantization Kernel in Triton", section 2: every block scale depends on the
// global scale, hence on the maximum over the entire rotated tensor).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "nvfp4rq_device.hpp"
#include "common.hpp"

namespace nvfp4rq {
namespace {  // one translation unit (nvfp4rq.hip): internal linkage

// Pass 1 for bf16.  Coalesced: in each
// iteration a wave reads 64 * kAmaxPieces consecutive 16-byte pieces, lane l
// taking pieces l, l + 64, ...; a piece is half a block, so lanes 2k and 2k+1
// hold elements 0..7 and 8..15 of one block.  Each lane runs the stride-1, 2,
// 4 stages on its half; the stride-8 stage pairs the two lanes, and
// max(|a + b|, |a - b|) = RN(|a| + |b|) exactly (rounding to nearest is
// symmetric), so one DPP-fed add per element gives the block's largest |z|.
// Both lanes compute the same sums; the maximum absorbs the duplicate.
// max |0.25 z| = RN(0.25 max |z|) because rounding is monotone, so the scaling
// is applied once at the end.
template <bool ROTATE>
__global__ __launch_bounds__(kThreads) void rotamax_bf16_kernel(const uint16_t* __restrict__ x,
                                                                int64_t nb,
                                                                uint32_t* __restrict__ amax_bits,
                                                                int partials, Counters counters,
                                                                int64_t nt_end) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = pass1_wg() * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (kThreads / 64);
  const int64_t npieces = 2 * nb;
  constexpr int64_t kPerWave = 64 * kAmaxPieces;
  const uint4* __restrict__ p = reinterpret_cast<const uint4*>(x);
  uint32_t m = 0u;
  for (int64_t base = wave * kPerWave; base < npieces; base += nwaves * kPerWave) {
    uint4 v[kAmaxPieces];
    if (base + kPerWave <= nt_end) {       // streamed past the caches (see launch_rotamax)
#pragma unroll
      for (int j = 0; j < kAmaxPieces; ++j) v[j] = load_nontemporal(p + base + j * 64 + lane);
    } else if (base + kPerWave <= npieces) {  // wave-uniform: every piece in range
#pragma unroll
      for (int j = 0; j < kAmaxPieces; ++j) v[j] = p[base + j * 64 + lane];
    } else {                               // the tensor's last, partial chunk
#pragma unroll
      for (int j = 0; j < kAmaxPieces; ++j) {
        const int64_t pc = base + j * 64 + lane;
        v[j] = pc < npieces ? p[pc] : make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int j = 0; j < kAmaxPieces; ++j) {
      float z[8];
      widen8(v[j], z);
      if (ROTATE) {
        stages_1_2_4(z);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          m = umax(m, __float_as_uint(__builtin_fabsf(z[i]) + __builtin_fabsf(swap_lane1(z[i]))));
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) m = umax(m, abs_bits(z[i]));
      }
    }
  }
  if (ROTATE) m = __float_as_uint(0.25f * __uint_as_float(m));
  workgroup_max_to(m, amax_bits, partials, counters);
}

// Pass 1 for fp32: one block per lane per iteration.
template <bool ROTATE>
__global__ __launch_bounds__(kThreads) void rotamax_f32_kernel(const float* __restrict__ x,
                                                               int64_t nb,
                                                               uint32_t* __restrict__ amax_bits,
                                                               int partials, Counters counters) {
  uint32_t m = 0u;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; b < nb; b += stride) {
    float lo[8], hi[8];
    load_block(x, b, lo, hi);
    if (ROTATE) {
      stages_1_2_4(lo);
      stages_1_2_4(hi);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        m = umax(m, __float_as_uint(__builtin_fabsf(lo[i]) + __builtin_fabsf(hi[i])));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) m = umax(umax(m, abs_bits(lo[i])), abs_bits(hi[i]));
    }
  }
  if (ROTATE) m = __float_as_uint(0.25f * __uint_as_float(m));
  workgroup_max_to(m, amax_bits, partials, counters);
}

}  // namespace
}  // namespace nvfp4rq
