// Kernels that write fp32 per element: decode (NVFP4 and MXFP4) and the
// rotation alone, in a quarter-block layout.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "nvfp4rq_device.hpp"
#include "common.hpp"
#include "pass2.hpp"

namespace nvfp4rq {
namespace {  // one translation unit (nvfp4rq.hip): internal linkage

// Kernels that write fp32 per element (decode, rotation alone) use a
// quarter-block layout: a wave takes 64 * kQuarters consecutive 4-element
// quarters per iteration, lane l quarters l, l + 64, ..., so that every store
// instruction of the wave writes 1 KiB of consecutive outputs.  A block's four
// quarters sit in the four lanes of a quad; strides 1 and 2 of the butterfly
// run in lane, strides 4 and 8 through quad lane exchanges, so every lane of
// a quad runs them, in partial iterations too (only loads and stores are
// predicated there).
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

// ---------------------------------------------------------------- decode

// The decode kernels give each wave one slice of kSliceQuarters consecutive
// quarters (2048 outputs) and launch one wave per slice.  A wave stages its
// slice's codes (1 KiB: two 8-byte loads per lane) and, for row-major scales,
// its scale bytes (one or two byte loads per lane) in its own part of LDS, and
// reads them back in the quarter layout.  Rotated decode at 16384 x 8192,
// event-timed around the kernel: 90 us like this; 109 us with per-quarter
// code and scale loads and one wave per slice; 124 us with per-quarter loads
// in a grid of 8 persistent workgroups per CU; the 512 MiB of fp32 stores
// alone, 79 us.
constexpr int64_t kSliceQuarters = 64 * kQuarters;

// Where a decode kernel finds the scale of a quarter and what a scale byte
// stands for.
template <typename SMAP>
struct Nvfp4Scales {  // one E4M3 byte per 16-element block: RN(float(s) * g)
  static constexpr int kQuartersPerScale = 4;
  // row-major: a slice's scale bytes are consecutive and are staged with its
  // codes; swizzled: each quarter reads its byte where the layout puts it
  static constexpr bool kStaged = std::is_same<SMAP, RowMajorScales>::value;
  SMAP smap;
  __device__ __forceinline__ int64_t index(int64_t block) const { return smap(block); }
  __device__ __forceinline__ float factor(uint32_t b, float g) const { return e4m3_value(b) * g; }
};
struct Mxfp4Scales {  // one E8M0 byte per 32-element block: 2^(byte - 127), exact
  static constexpr int kQuartersPerScale = 8;
  static constexpr bool kStaged = true;
  __device__ __forceinline__ int64_t index(int64_t block) const { return block; }
  __device__ __forceinline__ float factor(uint32_t b, float) const {
    return ldexpf(1.0f, static_cast<int>(b) - 127);
  }
};

// Hand-over through LDS inside one wave: the wave's stores are complete and
// visible to its own later loads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Decode (section 2, dequantize): +-GRID[c & 7] * scale factor, each product a
// binary32 multiply, then the same butterfly and * 0.25 when rotated (H16 is
// symmetric, so H16^T is the forward transform).  nq = number of quarters;
// gscale may be null for scales that need no global factor (MXFP4).
// TAIL = false: the waves take the nq / kSliceQuarters whole slices, with no
// bounds checks (a store burst broken up by per-lane guards costs 10% here);
// TAIL = true: one wave takes the partial slice at the end, if there is one.
template <typename SRC, bool ROTATE, bool TAIL>
__global__ __launch_bounds__(kThreads) void decode_kernel(const uint8_t* __restrict__ q,
                                                          const uint8_t* __restrict__ s,
                                                          const float* __restrict__ gscale,
                                                          int64_t nq, float* __restrict__ y, SRC src) {
  constexpr int kScaleBytes = static_cast<int>(kSliceQuarters) / SRC::kQuartersPerScale;
  __shared__ uint2 codes[kThreads / 64][kSliceQuarters / 4];
  __shared__ uint8_t scales[kThreads / 64][SRC::kStaged ? kScaleBytes : 1];
  const uint32_t lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t nslices = TAIL ? (nq % kSliceQuarters != 0) : nq / kSliceQuarters;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (blockDim.x / 64);
  uint16_t* c16 = reinterpret_cast<uint16_t*>(&codes[wv][0]);
  float4* __restrict__ o = reinterpret_cast<float4*>(y);
  const float g = gscale ? *gscale : 1.0f;
  for (int64_t w = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x * (blockDim.x / 64) + wv));
       w < nslices; w += nwaves) {
    const int64_t base = (TAIL ? nq / kSliceQuarters : w) * kSliceQuarters;
    const int64_t first = base / SRC::kQuartersPerScale;
    if (!TAIL) {
      const uint2* __restrict__ q8 = reinterpret_cast<const uint2*>(q);
      codes[wv][lane] = q8[(base >> 2) + lane];
      codes[wv][lane + 64] = q8[(base >> 2) + 64 + lane];
      if constexpr (SRC::kStaged) {
#pragma unroll
        for (int i = 0; i < kScaleBytes; i += 64) scales[wv][i + lane] = s[first + i + lane];
      }
    } else {
      const uint16_t* __restrict__ q2 = reinterpret_cast<const uint16_t*>(q);
      const int64_t nscales = nq / SRC::kQuartersPerScale;
#pragma unroll
      for (int j = 0; j < kQuarters; ++j) {
        const int64_t pc = base + j * 64 + lane;
        c16[j * 64 + lane] = pc < nq ? q2[pc] : uint16_t{0};
      }
      if constexpr (SRC::kStaged) {
#pragma unroll
        for (int i = 0; i < kScaleBytes; i += 64)
          scales[wv][i + lane] = first + i + lane < nscales ? s[first + i + lane] : uint8_t{0};
      }
    }
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < kQuarters; ++j) {
      const uint32_t qi = j * 64 + lane;
      const int64_t pc = base + qi;
      const uint32_t c = c16[qi];
      uint32_t sb;
      if constexpr (SRC::kStaged)
        sb = scales[wv][qi / SRC::kQuartersPerScale];
      else
        sb = (!TAIL || pc < nq) ? s[src.index(pc / SRC::kQuartersPerScale)] : 0u;
      const float f = src.factor(sb, g);
      const float2 v01 = e2m1_pair<0>(c), v23 = e2m1_pair<1>(c);
      float z[4] = {v01.x * f, v01.y * f, v23.x * f, v23.y * f};
      if (ROTATE) {
        stages_1_2(z);
        quad_stages_4_8(z, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = 0.25f * z[i];
      }
      if (!TAIL || pc < nq) o[pc] = make_float4(z[0], z[1], z[2], z[3]);
    }
    wave_lds_sync();  // the slice's LDS is rewritten by the next iteration
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

// ---------------------------------------------------------------- general rotation

// Lane s of the quad, broadcast to the whole quad (quad_perm [s, s, s, s]).
template <int S>
__device__ __forceinline__ float quad_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), S * 0x55, 0xF, 0xF, false));
}

// y = x r for every 16-element block (r: 16 x 16 binary32, row-major, rows
// are inputs): the Hadamard replaced by a general matrix, as the page "A
// Fused Hadamard + NVFP4 Quantization Kernel in Triton" proposes in its "Try
// this" item 3 (a random orthogonal matrix).  Quarter-block layout: each lane
// gathers its block's 16 inputs from the quad by broadcasts and computes its
// four outputs y_j = RN(x_0 r_0j), then fused multiply-adds in k order, the
// summation order the reading fixes.  r is staged in LDS.
template <typename T>
__global__ __launch_bounds__(kThreads) void rotate_matrix_kernel(const T* __restrict__ x, int64_t nq,
                                                                 const float* __restrict__ r,
                                                                 float* __restrict__ y) {
  __shared__ float4 rs[64];  // row k, columns 4c .. 4c + 3 at rs[4k + c]
  if (threadIdx.x < 64) rs[threadIdx.x] = reinterpret_cast<const float4*>(r)[threadIdx.x];
  __syncthreads();
  const uint32_t lane = threadIdx.x & 63, t = lane & 3u;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (kThreads / 64);
  constexpr int64_t kPerWave = 64 * kQuarters;
  float4* __restrict__ o = reinterpret_cast<float4*>(y);
  for (int64_t base = wave * kPerWave; base < nq; base += nwaves * kPerWave) {
#pragma unroll 2
    for (int j = 0; j < kQuarters; ++j) {
      const int64_t pc = base + j * 64 + lane;
      float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (pc < nq) load_quarter(x, pc, z);
      float xs[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xs[i] = quad_bcast<0>(z[i]);
        xs[4 + i] = quad_bcast<1>(z[i]);
        xs[8 + i] = quad_bcast<2>(z[i]);
        xs[12 + i] = quad_bcast<3>(z[i]);
      }
      const float4 r0 = rs[t];
      float4 acc = make_float4(xs[0] * r0.x, xs[0] * r0.y, xs[0] * r0.z, xs[0] * r0.w);
#pragma unroll
      for (int k = 1; k < 16; ++k) {
        const float4 rk = rs[4 * k + t];
        acc.x = __builtin_fmaf(xs[k], rk.x, acc.x);
        acc.y = __builtin_fmaf(xs[k], rk.y, acc.y);
        acc.z = __builtin_fmaf(xs[k], rk.z, acc.z);
        acc.w = __builtin_fmaf(xs[k], rk.w, acc.w);
      }
      if (pc < nq) o[pc] = acc;
    }
  }
}

}  // namespace
}  // namespace nvfp4rq
