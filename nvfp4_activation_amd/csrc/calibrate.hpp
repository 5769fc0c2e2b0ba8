// Measurement support, not part of the method: twins of the fused call's two
// kernels that move the same bytes in the same access patterns and launch
// shapes (grid, wave layout, non-temporal rule, chunk order, store widths) and
// do no arithmetic beyond a bitwise fold that keeps every load alive.  Timing
// them gives the ceiling the call's byte mix can reach on the machine at hand.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.hpp"
#include "pass2.hpp"

namespace nvfp4rq {
namespace {  // one translation unit (nvfp4rq.hip): internal linkage

__device__ __forceinline__ uint32_t fold(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Twin of rotamax_bf16_kernel: the same loop over 16-byte pieces; the
// workgroup's fold goes where pass 1 puts its maximum.
__global__ __launch_bounds__(kThreads) void stream_read_bf16_kernel(const uint16_t* __restrict__ x,
                                                                    int64_t nb,
                                                                    uint32_t* __restrict__ out,
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
    if (base + kPerWave <= nt_end) {
#pragma unroll
      for (int j = 0; j < kAmaxPieces; ++j) v[j] = load_nontemporal(p + base + j * 64 + lane);
    } else if (base + kPerWave <= npieces) {
#pragma unroll
      for (int j = 0; j < kAmaxPieces; ++j) v[j] = p[base + j * 64 + lane];
    } else {
#pragma unroll
      for (int j = 0; j < kAmaxPieces; ++j) {
        const int64_t pc = base + j * 64 + lane;
        v[j] = pc < npieces ? p[pc] : make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int j = 0; j < kAmaxPieces; ++j) m ^= fold(v[j]);
  }
  workgroup_max_to(m, out, partials, counters);
}

// Twin of rotamax_f32_kernel: one 64-byte block per lane per iteration.
__global__ __launch_bounds__(kThreads) void stream_read_f32_kernel(const float* __restrict__ x,
                                                                   int64_t nb,
                                                                   uint32_t* __restrict__ out,
                                                                   int partials, Counters counters) {
  uint32_t m = 0u;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; b < nb; b += stride) {
    const uint4* p = reinterpret_cast<const uint4*>(x + b * 16);
    m ^= fold(p[0]) ^ fold(p[1]) ^ fold(p[2]) ^ fold(p[3]);
  }
  workgroup_max_to(m, out, partials, counters);
}

// Twin of rotquant_kernel with row-major scales: the same chunk order and
// raw buffer accesses; each lane loads its block, stores 8 bytes
// non-temporally where its codes go and one byte where its scale goes.
template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void stream_rw_kernel(
    const T* __restrict__ x, int64_t nb, uint8_t* q, uint8_t* s, RowMajorScales smap, Launch vis) {
  const uint32_t nchunks = vis.nchunks;
  const uint32_t nfull = static_cast<uint32_t>(nb / kThreads);
  const uint32_t tail = static_cast<uint32_t>(nb % kThreads);
  const uint32_t mine = vis.of(blockIdx.x);
  for (int32_t it = static_cast<int32_t>(mine) - 1; it >= 0; --it) {
    const uint32_t chunk = smap.order(static_cast<uint32_t>(it) * vis.grid + blockIdx.x, nchunks);
    const uint32_t valid = chunk < nfull ? kThreads : tail;
    Block<T> blk;
    blk.load(x, chunk, valid, threadIdx.x);
    uint32_t w0, w1;
    if constexpr (sizeof(T) == 2) {
      w0 = blk.a.x ^ blk.a.y ^ blk.a.z ^ blk.a.w;
      w1 = blk.b.x ^ blk.b.y ^ blk.b.z ^ blk.b.w;
    } else {
      w0 = blk.a.x ^ blk.a.y ^ blk.a.z ^ blk.a.w ^ blk.b.x ^ blk.b.y ^ blk.b.z ^ blk.b.w;
      w1 = blk.c.x ^ blk.c.y ^ blk.c.z ^ blk.c.w ^ blk.d.x ^ blk.d.y ^ blk.d.z ^ blk.d.w;
    }
    store_chunk_block(q, s, chunk, valid, threadIdx.x, u32x2{w0, w1}, w0 ^ w1);
  }
}

}  // namespace
}  // namespace nvfp4rq
