// Launch constants, reductions and block loads shared by the kernels of
// libnvfp4rq (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "nvfp4rq_device.hpp"

namespace nvfp4rq {
namespace {  // one translation unit (nvfp4rq.hip): internal linkage

constexpr int kThreads = 256;      // 4 waves of 64
// 16-byte pieces per lane per iteration in the bf16 amax pass: 4 KiB per
// wave.  Against 8: pass 1 at 16384 x 8192 42.0 instead of 44.9 us, at
// 32768 x 14336 132 instead of 141 us; 2 and 16 were slower than both.
constexpr int kAmaxPieces = 4;

// The fast path (corrected divisions with per-scale reciprocals) is used for
// bf16 input when the global amax lies in [2^-38, 2^15): then every divisor is
// in [2^-58.4, 2^14.4] and every quotient stays inside the range on which the
// corrected division was enumerated.  Other tensors take the exact path
// (IEEE divisions); both give identical bytes.
constexpr uint32_t kFastAmaxLo = 0x2C800000u;   // 2^-38
constexpr uint32_t kFastAmaxHi = 0x47000000u;   // 2^15
// Corrected divisions stay finite while |z| / d <= 2^100; larger quotients
// (possible only when the global scale comes from another tensor's amax) take
// true divisions.
constexpr float kQuotientLimit = 0x1p100f;
constexpr int64_t kLastLevelKeep = 160LL << 20;  // bytes of input pass 1 leaves cached
// From this input size on, the two passes of a row-major call hand the amax
// over through a zeroed word instead of per-workgroup maxima, so that pass 2
// can run a workgroup per chunk (see enqueue_both).
constexpr int64_t kOneShotInputBytes = 512LL << 20;
// When pass 1 leaves its per-workgroup maxima in the outputs (the head), they
// sit at words [0, grid) of kMaxPartials (pass 1's grid is at most that, and
// its workgroup 0 clears the words from grid on), and the quantize
// pass's arrival counters are kCounters words on separate 128-byte lines
// (thousands of increments of one word serialize, and a workgroup's loads
// wait behind its own pending atomic).  Row-major scales: both in q_out, the
// maxima in chunk 0's 2 KiB of codes and the counters in chunk 1's, kHeadBytes
// in all.  Swizzled scales: the maxima in chunk 0's 2 KiB of scale tiles, the
// counters at the start of code rows 0 .. kCounters - 1, also chunk 0's.
// Only the quantize workgroup that writes the head's chunks reads the
// counters, and it writes those chunks last, after its wait: nothing
// overwrites a counter that is still being read.
constexpr int kMaxPartials = 512;
constexpr int kCounters = 16;
constexpr int kCounterStride = 32;                                               // words (row-major)
constexpr int64_t kCounterBase = kMaxPartials;                                   // words (row-major)
constexpr int64_t kHeadBytes = 4 * (kCounterBase + kCounters * kCounterStride);  // 4096

// Where the arrival counters are: kCounters words, `stride` words apart.
struct Counters {
  uint32_t* base;
  uint32_t stride;
  __host__ __device__ uint32_t* at(uint32_t i) const { return base + static_cast<int64_t>(i) * stride; }
};

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Logical workgroup index of the bf16 amax pass.  Workgroups go round-robin
// to the 8 XCDs (XCD b % 8), and a logical workgroup iteration reads
// kAmaxPieces / 2 = 2 chunks of 256 blocks.  Physical workgroup b, the j-th on
// its XCD (j = b / 8), becomes 16 (j / 2) + 2 (b % 8) + j % 2, so each XCD
// reads runs of 4 consecutive chunks: chunk c on XCD (c / 4) % 8, the XCD on
// which the quantize pass's order visits it (RowMajorScales::order), which
// then finds it in that XCD's L2 (16384 x 8192 step: 98.6 -> 97.5 us;
// 4096 x 4096: 21.4 -> 20.2 us).  A bijection when the grid is a multiple of
// 16; other grids keep b.
static_assert(kAmaxPieces == 4, "pass1_wg pairs workgroups of two chunks each");
__host__ __device__ inline int64_t pass1_wg_of(int64_t b, int64_t grid) {
  if (grid % 16 != 0) return b;
  const int64_t j = b >> 3;
  return 16 * (j >> 1) + 2 * (b & 7) + (j & 1);
}
__device__ __forceinline__ int64_t pass1_wg() { return pass1_wg_of(blockIdx.x, gridDim.x); }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t u) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(u), CTRL, 0xF, 0xF, false));
}

// Wave maximum as a wave-uniform (scalar) value: each row of 16 lanes by DPP
// exchanges (quad_perm [1,0,3,2] and [2,3,0,1], then the half-row and row
// mirrors), then the four rows through readlane.  No LDS round trips.  Every
// lane of the wave must be active.
__device__ __forceinline__ uint32_t wave_max_u32_uniform(uint32_t u) {
  u = umax(u, dpp_u32<0xB1>(u));
  u = umax(u, dpp_u32<0x4E>(u));
  u = umax(u, dpp_u32<0x141>(u));
  u = umax(u, dpp_u32<0x140>(u));
  const uint32_t r0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u), 0));
  const uint32_t r1 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u), 16));
  const uint32_t r2 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u), 32));
  const uint32_t r3 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u), 48));
  return umax(umax(r0, r1), umax(r2, r3));
}

// Sum of lanes 0..15 (the wave's first row) as a wave-uniform value: the same
// DPP exchanges with additions, then readlane 0.  Every lane of the wave must
// be active.
__device__ __forceinline__ uint32_t row0_sum_u32(uint32_t u) {
  u += dpp_u32<0xB1>(u);
  u += dpp_u32<0x4E>(u);
  u += dpp_u32<0x141>(u);
  u += dpp_u32<0x140>(u);
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u), 0));
}

// Workgroup maximum, then either one atomicMax per workgroup on a zeroed word
// (partials == 0), or a plain store of the workgroup's maximum to out[wg]
// (partials == 1; workgroup 0 also clears the arrival counters the quantize
// pass uses, so no word has to be zeroed beforehand, and the words from
// out[grid] to out[kMaxPartials - 1], so that the quantize pass reduces all
// kMaxPartials words without masking).  Non-negative binary32 values order
// like their bit patterns, so the maximum is exact and the same for any
// reduction order (a NaN input stays visible as bits above +inf).  Every
// thread of the workgroup must call it.
__device__ __forceinline__ void workgroup_max_to(uint32_t m, uint32_t* __restrict__ out,
                                                 int partials, Counters counters) {
  __shared__ uint32_t part[kThreads / 64];
  m = wave_max_u32_uniform(m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = part[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) r = umax(r, part[i]);
    if (partials)
      out[blockIdx.x] = r;
    else
      atomicMax(out, r);
  }
  if (partials && blockIdx.x == 0) {
    if (threadIdx.x < kCounters) *counters.at(threadIdx.x) = 0u;
    for (uint32_t i = gridDim.x + threadIdx.x; i < static_cast<uint32_t>(kMaxPartials); i += kThreads)
      out[i] = 0u;
  }
}

__device__ __forceinline__ uint32_t abs_bits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

__global__ void zero_word_kernel(uint32_t* __restrict__ w) { *w = 0u; }

// Raw buffer resources: a base address and a size in bytes; the address
// arithmetic stays in scalar registers, and lanes whose offset falls past the
// size load zeros and have their stores dropped by the hardware's range
// check.
constexpr int kBufferWord3 = 0x00020000;  // gfx9 raw buffer, 32-bit data format
constexpr int kNontemporal = 2;           // cache-policy bit of a non-temporal access

__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           kBufferWord3);
}

// Non-temporal loads and stores: data that no later pass will find in (or
// should take from) the caches.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_nontemporal(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// One 16-value fp32 block: elements 0..7 into lo, 8..15 into hi.
__device__ __forceinline__ void load_block(const float* __restrict__ x, int64_t b, float lo[8],
                                           float hi[8]) {
  const float4* p = reinterpret_cast<const float4*>(x + b * 16);
  const float4 a = p[0], c = p[1], d = p[2], e = p[3];
  lo[0] = a.x; lo[1] = a.y; lo[2] = a.z; lo[3] = a.w;
  lo[4] = c.x; lo[5] = c.y; lo[6] = c.z; lo[7] = c.w;
  hi[0] = d.x; hi[1] = d.y; hi[2] = d.z; hi[3] = d.w;
  hi[4] = e.x; hi[5] = e.y; hi[6] = e.z; hi[7] = e.w;
}

// One 16-value bf16 block (32 bytes), widened.
__device__ __forceinline__ void load_block(const uint16_t* __restrict__ x, int64_t b, float lo[8],
                                           float hi[8]) {
  const uint4* p = reinterpret_cast<const uint4*>(x + b * 16);
  widen8(p[0], lo);
  widen8(p[1], hi);
}

}  // namespace
}  // namespace nvfp4rq
