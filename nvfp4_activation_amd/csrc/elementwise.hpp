// Kernels that write fp32 per element: decode (NVFP4 and MXFP4) and the
// rotation alone, in a quarter-block layout.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "nvfp4rq_device.hpp"
#include "common.hpp"

namespace nvfp4rq {
namespace {  // one translation unit (nvfp4rq.hip): internal linkage

// Kernels that write fp32 per element (decode, rotation alone) use a
// quarter-block layout: a wave takes 64 * kQuarters consecutive 4-element
// quarters per iteration, lane l quarters l, l + 64, ..., so that every store
// instruction of the wave writes 1 KiB of consecutive outputs.  A block's four
// quarters sit in the four lanes of a quad; strides 1 and 2 of the butterfly
// run in lane, strides 4 and 8 through quad lane exchanges.  The tail
// iteration is wave-uniform and every lane runs the exchanges; only the loads
// and stores are predicated.
constexpr int kQuarters = 8;

__device__ __forceinline__ void load_quarter(const float* __restrict__ x, int64_t pc, float z[4]) {
  const float4 v = reinterpret_cast<const float4*>(x)[pc];
  z[0] = v.x; z[1] = v.y; z[2] = v.z; z[3] = v.w;
}

__device__ __forceinline__ void load_quarter(const uint16_t* __restrict__ x, int64_t pc,
                                             float z[4]) {
  const uint2 v = reinterpret_cast<const uint2*>(x)[pc];
  z[0] = bf16_lo(v.x); z[1] = bf16_hi(v.x); z[2] = bf16_lo(v.y); z[3] = bf16_hi(v.y);
}

// Dequantize (section 2, dequantize): +-GRID[c & 7] * RN(float(s) * g), then
// the same butterfly and * 0.25 when rotated (H16 is symmetric, so H16^T is
// the forward transform).  nq = number of quarters = rows * cols / 4.
template <typename SMAP>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* __restrict__ q,
                                                           const uint8_t* __restrict__ s,
                                                           const float* __restrict__ gscale,
                                                           int64_t nq, int rotate,
                                                           float* __restrict__ y, SMAP smap) {
  const uint32_t lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (kThreads / 64);
  constexpr int64_t kPerWave = 64 * kQuarters;
  const uint16_t* __restrict__ q2 = reinterpret_cast<const uint16_t*>(q);  // 4 codes
  float4* __restrict__ o = reinterpret_cast<float4*>(y);
  const float g = *gscale;
  for (int64_t base = wave * kPerWave; base < nq; base += nwaves * kPerWave) {
    uint32_t c[kQuarters], sb[kQuarters];
#pragma unroll
    for (int j = 0; j < kQuarters; ++j) {
      const int64_t pc = base + j * 64 + lane;
      const bool in = pc < nq;
      c[j] = in ? q2[pc] : 0u;
      sb[j] = in ? s[smap(pc >> 2)] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kQuarters; ++j) {
      const float sf = e4m3_value(sb[j]) * g;
      float z[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) z[i] = e2m1_value((c[j] >> (4 * i)) & 15u) * sf;
      if (rotate) {
        stages_1_2(z);
        quad_stages_4_8(z, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = 0.25f * z[i];
      }
      const int64_t pc = base + j * 64 + lane;
      if (pc < nq) o[pc] = make_float4(z[0], z[1], z[2], z[3]);
    }
  }
}

// ---------------------------------------------------------------- rotation alone

// y = x H16 per 16-element block (butterfly, then * 0.25), stored as fp32.
// The first kernel of the unfused three-kernel arrangement that the page
// "A Fused Hadamard + NVFP4 Quantization Kernel in Triton" compares the fused
// kernel against (opening paragraph; "Try this" item 4): rotated values go to
// HBM and the amax and quantize kernels read them back with rotation off.
template <typename T>
__global__ __launch_bounds__(kThreads) void rotate_kernel(const T* __restrict__ x, int64_t nq,
                                                          float* __restrict__ y) {
  const uint32_t lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (kThreads / 64);
  constexpr int64_t kPerWave = 64 * kQuarters;
  float4* __restrict__ o = reinterpret_cast<float4*>(y);
  for (int64_t base = wave * kPerWave; base < nq; base += nwaves * kPerWave) {
    float z[kQuarters][4];
    if (base + kPerWave <= nq) {           // wave-uniform: every quarter in range
#pragma unroll
      for (int j = 0; j < kQuarters; ++j) load_quarter(x, base + j * 64 + lane, z[j]);
    } else {
#pragma unroll
      for (int j = 0; j < kQuarters; ++j) {
        const int64_t pc = base + j * 64 + lane;
        if (pc < nq) {
          load_quarter(x, pc, z[j]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) z[j][i] = 0.0f;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kQuarters; ++j) {
      stages_1_2(z[j]);
      quad_stages_4_8(z[j], lane);
      const int64_t pc = base + j * 64 + lane;
      if (pc < nq)
        o[pc] = make_float4(0.25f * z[j][0], 0.25f * z[j][1], 0.25f * z[j][2], 0.25f * z[j][3]);
    }
  }
}

// MXFP4 dequantize: +-GRID[c & 7] * 2^(byte - 127), rounded to binary32, then
// the inverse rotation of each 16-element half (the same butterfly and
// * 0.25).  Quarter-block layout as for the NVFP4 decode; a 32-element block
// is two quads.
__global__ __launch_bounds__(kThreads) void mx_dequant_kernel(const uint8_t* __restrict__ q,
                                                              const uint8_t* __restrict__ s,
                                                              int64_t nq, int rotate,
                                                              float* __restrict__ y) {
  const uint32_t lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (kThreads / 64);
  constexpr int64_t kPerWave = 64 * kQuarters;
  const uint16_t* __restrict__ q2 = reinterpret_cast<const uint16_t*>(q);
  float4* __restrict__ o = reinterpret_cast<float4*>(y);
  for (int64_t base = wave * kPerWave; base < nq; base += nwaves * kPerWave) {
    uint32_t c[kQuarters], sb[kQuarters];
#pragma unroll
    for (int j = 0; j < kQuarters; ++j) {
      const int64_t pc = base + j * 64 + lane;
      const bool in = pc < nq;
      c[j] = in ? q2[pc] : 0u;
      sb[j] = in ? s[pc >> 3] : 127u;
    }
#pragma unroll
    for (int j = 0; j < kQuarters; ++j) {
      const float sc = ldexpf(1.0f, static_cast<int>(sb[j]) - 127);
      float z[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) z[i] = e2m1_value((c[j] >> (4 * i)) & 15u) * sc;
      if (rotate) {
        stages_1_2(z);
        quad_stages_4_8(z, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = 0.25f * z[i];
      }
      const int64_t pc = base + j * 64 + lane;
      if (pc < nq) o[pc] = make_float4(z[0], z[1], z[2], z[3]);
    }
  }
}

}  // namespace
}  // namespace nvfp4rq
