// Pass 2: global scale, rotation, block scales and E2M1 codes (page "A Fused
// Hadamard + NVFP4 Quantization Kernel in Triton", section 2,
// hadamard_nvfp4_kernel), in row-major or swizzled scale layout.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "nvfp4rq_device.hpp"
#include "common.hpp"

namespace nvfp4rq {
namespace {  // one translation unit (nvfp4rq.hip): internal linkage

// Where block b's scale byte is stored.  Row-major: byte b of the
// [rows, cols/16] matrix.  Swizzled (the tiled layout GEMMs read, page "A
// Fused Hadamard + NVFP4 Quantization Kernel in Triton", section 6; layout as
// the GEMM library documentation it cites defines it for 16-element block
// scales): the matrix padded to 128-row x 4-column tiles of 512 bytes, tiles
// stored tile-row by tile-row, and S[128 rt + 32 i + j][4 ct + k] at byte
// 512 (rt * ctiles + ct) + 16 j + 4 i + k.  Block indices fit in 32 bits
// (checked on the host).
// Each policy also fixes which blocks a pass-2 workgroup handles together
// (a chunk): kSub groups of kThreads blocks.  Row-major: 256 consecutive
// blocks.  Swizzled: a super-tile of 128 rows x 16 blocks, so that one
// workgroup writes whole 512-byte scale tiles and whole 128-byte lines of
// codes (lines completed from several L2s are written back piecemeal).
struct RowMajorScales {
  static constexpr int kSub = 1;
  static constexpr bool kStaged = false;
  int xcd_order;  // give each XCD runs of 4 consecutive chunks
  int mirror;     // a workgroup per chunk, workgroup i taking chunk nchunks - 1 - i
  __device__ __forceinline__ int64_t operator()(int64_t b) const { return b; }
  __host__ __device__ int64_t chunks(int64_t nb) const { return (nb + kThreads - 1) / kThreads; }
  // Workgroups go round-robin to the 8 XCDs, each with its own L2 and address
  // translation caches.  The order gives each XCD runs of 4 consecutive
  // chunks (32 KiB of bf16 input): visit index i runs on XCD i % 8 and takes
  // chunk (i & ~31) | ((i & 7) << 2) | ((i >> 3) & 3), a permutation within
  // each group of 32 chunks.  The bf16 amax pass reads chunk c on XCD
  // (c / 4) % 8 too (pass1_wg), so the chunks it read last are still in the
  // visiting XCD's L2.  The run length pays by itself as well: before the
  // amax pass matched it, pass 2 at 16384 x 8192 took 56.2, 55.2, 53.3 and
  // 53.3 us with runs of 1, 2, 4 and 8 chunks on one box, and 53.5, 54.0,
  // 54.0, 54.9 and 57.2 us with runs of 4, 8, 16, 64 and 256 on another.
  // Set only when the chunk count is a multiple of 32.
  // With a workgroup per chunk the dispatcher starts workgroups in index
  // order, so mirror keeps the last chunks (the likeliest to be still cached
  // after an amax pass) first.
  __device__ __forceinline__ int64_t order(int64_t i, int64_t nchunks) const {
    if (mirror) return nchunks - 1 - i;
    return xcd_order ? (i & ~int64_t{31}) | ((i & 7) << 2) | ((i >> 3) & 3) : i;
  }
  __device__ __forceinline__ bool locate(int64_t chunk, int, uint32_t tid, int64_t nb, int64_t* b,
                                         int64_t* si) const {
    *b = chunk * kThreads + tid;
    *si = *b;
    return *b < nb;
  }
};
struct SwizzledScales {
  static constexpr int kSub = 8;
  static constexpr bool kStaged = true;  // scale tiles assembled in LDS
  int64_t rows;
  uint32_t cb, ctiles, cs;  // blocks per row, ceil(cb / 4), ceil(cb / 16)
  int mirror;               // as RowMajorScales::mirror
  int runs16;               // give each XCD runs of 16 consecutive chunks
  // A chunk's row tile and 16-block column, divided out once per chunk (a
  // 64-bit division per sub-iteration cost 135 scalar instructions each).
  struct Tile {
    int64_t rt;
    uint32_t cw;
  };
  __device__ __forceinline__ Tile split(int64_t chunk) const {
    const int64_t rt = chunk / cs;
    return Tile{rt, static_cast<uint32_t>(chunk - rt * cs)};
  }
  __device__ __forceinline__ static int64_t place(uint32_t r, uint32_t c, uint32_t ctiles) {
    const uint64_t tile = static_cast<uint64_t>(r >> 7) * ctiles + (c >> 2);
    return static_cast<int64_t>(tile * 512u + (((r & 31u) << 4) | (((r >> 5) & 3u) << 2) | (c & 3u)));
  }
  __device__ __forceinline__ int64_t operator()(int64_t b) const {
    const uint32_t bb = static_cast<uint32_t>(b);
    const uint32_t r = bb / cb;
    return place(r, bb - r * cb, ctiles);
  }
  __host__ __device__ int64_t chunks(int64_t) const { return ((rows + 127) / 128) * cs; }
  // runs16: visit index i (on XCD i % 8) takes chunk (i & ~127) | ((i & 7)
  // << 4) | ((i >> 3) & 15), so each XCD reads 16 consecutive column windows
  // of a row tile (8 KiB of every bf16 row) instead of one.  Step at
  // 16384 x 8192: 101.5 us against 106.7 in plain order (runs of 2, 4, 8, 32,
  // 64: 122.5, 106.6, 115.4, 101.7, 101.2 us); 4096 x 4096: 22.2 against
  // 23.6 us.  Used when a row tile holds a multiple of 16 windows (at
  // 32768 x 14336, 56 windows, runs of 16 cost 2.7%) and the chunk count is a
  // multiple of 128.
  __device__ __forceinline__ int64_t order(int64_t i, int64_t nchunks) const {
    if (mirror) return nchunks - 1 - i;
    return runs16 ? (i & ~int64_t{127}) | ((i & 7) << 4) | ((i >> 3) & 15) : i;
  }
  __device__ __forceinline__ bool locate(Tile t, int sub, uint32_t tid, int64_t* b, int64_t* si) const {
    const uint32_t r = static_cast<uint32_t>(t.rt * 128 + sub * 16 + (tid >> 4));
    const uint32_t c = t.cw * 16 + (tid & 15u);
    if (r >= rows || c >= cb) return false;
    *b = static_cast<int64_t>(r) * cb + c;
    *si = place(r & 127u, c & 15u, 4);  // byte within the chunk's tiles
    return true;
  }
  // The chunk's tiles (rt, 4 cw .. 4 cw + 3) are consecutive in memory.
  __device__ __forceinline__ void chunk_tiles(Tile t, int64_t* first_byte, int* ntiles) const {
    const int64_t ct0 = static_cast<int64_t>(t.cw) * 4;
    *first_byte = (t.rt * ctiles + ct0) * 512;
    *ntiles = static_cast<int>(ctiles - ct0 < 4 ? ctiles - ct0 : 4);
  }
};

// When pass 1 leaves its per-workgroup maxima at the head of q_out (chunk 0,
// with the arrival counters in chunk 1), every pass-2 workgroup reads them in
// its prologue and then counts itself in.  One workgroup alone, the one that
// draws chunk 0, waits for all of them to have done so and then writes both
// head chunks; nobody else waits, so the count always completes, and no
// counter is written over while another workgroup still reads it.  Chunks run
// last-first, so that wait comes at the end of its workgroup.  It is bounded:
// past spin_limit sleeps the workgroup goes on and marks the call failed with
// a NaN global scale.
struct HeadGuard {
  uint32_t* counters;  // null: no maxima in q_out
  uint32_t need;       // quantize workgroups
  uint32_t spin_limit;
  float* gscale_out;
};

__device__ __forceinline__ void wait_for_head(const HeadGuard& h) {
  __shared__ int timed_out;
  if (threadIdx.x < 64) {  // wave 0: one counter per lane (lanes past kCounters add 0)
    uint32_t spins = 0;
    int late = 0;
    // Each poll reads a counter with a fetch-and-add of zero: an atomic,
    // performed where the increments are performed, so no copy of the line
    // in another cache can answer it.  Relaxed ordering: acquire/release at agent scope would write back or
    // invalidate the L2 of every XCD involved on each poll.  Nothing written
    // by other workgroups is read after the wait; the waiter's stores follow
    // the loop.
    // The compiler turns an add of a literal 0 back into a load, so the zero
    // is made opaque to it (an empty asm statement that only claims to
    // change the register).
    uint32_t zero = 0u;
    __asm__ volatile("" : "+v"(zero));
    for (;;) {
      uint32_t c = threadIdx.x < kCounters
                       ? __hip_atomic_fetch_add(h.counters + threadIdx.x * kCounterStride, zero,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                       : 0u;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) c += static_cast<uint32_t>(__shfl_xor(static_cast<int>(c), off, 64));
      if (c >= h.need) break;
      if (++spins > h.spin_limit) {
        late = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (threadIdx.x == 0) timed_out = late;
  }
  __syncthreads();
  if (timed_out && threadIdx.x == 0) *h.gscale_out = __uint_as_float(0x7FC00000u);
}

// A lane's first block, loaded (as raw bits) before the kernel's prologue so
// that the load latency overlaps the amax reduction and the table set-up.
template <typename T>
struct FirstBlock;
template <>
struct FirstBlock<uint16_t> {
  uint4 a, b;
  __device__ __forceinline__ void load(const uint16_t* x, int64_t blk) {
    const uint4* p = reinterpret_cast<const uint4*>(x + blk * 16);
    a = p[0];
    b = p[1];
  }
  __device__ __forceinline__ void unpack(float lo[8], float hi[8]) const {
    widen8(a, lo);
    widen8(b, hi);
  }
};
template <>
struct FirstBlock<float> {
  float4 a, b, c, d;
  __device__ __forceinline__ void load(const float* x, int64_t blk) {
    const float4* p = reinterpret_cast<const float4*>(x + blk * 16);
    a = p[0];
    b = p[1];
    c = p[2];
    d = p[3];
  }
  __device__ __forceinline__ void unpack(float lo[8], float hi[8]) const {
    lo[0] = a.x; lo[1] = a.y; lo[2] = a.z; lo[3] = a.w;
    lo[4] = b.x; lo[5] = b.y; lo[6] = b.z; lo[7] = b.w;
    hi[0] = c.x; hi[1] = c.y; hi[2] = c.z; hi[3] = c.w;
    hi[4] = d.x; hi[5] = d.y; hi[6] = d.z; hi[7] = d.w;
  }
};

template <typename T, typename SMAP>
__device__ __forceinline__ void load_first(const T* __restrict__ x, int64_t nb, SMAP smap,
                                           FirstBlock<T>* f) {
  const int64_t nchunks = smap.chunks(nb);
  const int64_t mine = (nchunks - blockIdx.x + gridDim.x - 1) / gridDim.x;
  int64_t b, si;
  if (mine > 0 && smap.locate(smap.order((mine - 1) * gridDim.x + blockIdx.x, nchunks), 0,
                              threadIdx.x, nb, &b, &si))
    f->load(x, b);
}

// The lane's block of the workgroup's second chunk (bf16, row-major), loaded
// before the prologue straight into LDS (the kernel has no registers to spare
// for it), 8 KiB per workgroup: 16384 x 8192 step 97.5 -> 95.7 us, pass 2
// 52.6 -> 51.1 us (three A/B pairs).  Used from 3 chunks per workgroup: with
// 2 (4096 x 4096) the prologue, whose wait for the maxima also waits for
// these loads, made the step 0.25 us slower.  quant_blocks_rm reads the
// block back under the same condition.
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;
__device__ __forceinline__ bool prefetches_second(int64_t mine) { return mine >= 3; }
__device__ __forceinline__ void prefetch_second(const uint16_t* __restrict__ x, int64_t nb,
                                                RowMajorScales smap, uint4* pre) {
  const int64_t nchunks = smap.chunks(nb);
  const int64_t mine = (nchunks - blockIdx.x + gridDim.x - 1) / gridDim.x;
  if (!prefetches_second(mine)) return;
  const int64_t b = smap.order((mine - 2) * gridDim.x + blockIdx.x, nchunks) * kThreads + threadIdx.x;
  if (b >= nb) return;
  const uint4* p = reinterpret_cast<const uint4*>(x + b * 16);
  // pre holds the blocks' first halves at [0, kThreads) and their second
  // halves at [kThreads, 2 kThreads).  The destination operand is per wave:
  // lane l's 16 bytes land at slot 64 w + l, i.e. at threadIdx.x.
  // Address-space conversions take C-style casts.
  const int w = threadIdx.x >> 6;
  __builtin_amdgcn_global_load_lds((global_void_ptr)(p), (lds_void_ptr)(pre + w * 64), 16, 0, 0);
  __builtin_amdgcn_global_load_lds((global_void_ptr)(p + 1), (lds_void_ptr)(pre + kThreads + w * 64), 16, 0,
                                   0);
}

// Swizzled chunks: the lane's block of the first sub-iteration of the
// workgroup's first chunk, loaded into LDS before the prologue (the pass has
// no registers to spare for the row-major pass's early first-block load):
// 16384 x 8192 swizzled step 101.3 -> 100.65 us, three A/B pairs.
__device__ __forceinline__ void prefetch_first_sw(const uint16_t* __restrict__ x, int64_t nb,
                                                  SwizzledScales smap, uint4* pre) {
  const int64_t nchunks = smap.chunks(nb);
  const int64_t mine = (nchunks - blockIdx.x + gridDim.x - 1) / gridDim.x;
  if (mine < 1) return;
  int64_t b, si;
  if (!smap.locate(smap.split(smap.order((mine - 1) * gridDim.x + blockIdx.x, nchunks)), 0, threadIdx.x, &b,
                   &si))
    return;
  const uint4* p = reinterpret_cast<const uint4*>(x + b * 16);
  const int w = threadIdx.x >> 6;
  __builtin_amdgcn_global_load_lds((global_void_ptr)(p), (lds_void_ptr)(pre + w * 64), 16, 0, 0);
  __builtin_amdgcn_global_load_lds((global_void_ptr)(p + 1), (lds_void_ptr)(pre + kThreads + w * 64), 16, 0,
                                   0);
}

// One block of pass 2, in one lane: rotation (in place on lo, hi), the block
// scale byte and the two words of E2M1 codes.  Every step is the definition
// of section 2 (hadamard_nvfp4_kernel) in binary32:
//   z     = S16 x                         (butterfly, no scaling yet)
//   a_b   = max |y| = 0.25 max |z|        (exact for any rounding, see pass 1)
//   v     = (a_b / 6) / g,  s = E4M3(min(v, 448))
//   d     = float(s) * g, or 1 when that is 0
//   code  = E2M1(y / d),  y = 0.25 z
// FAST (bf16 in the guarded range): y / d = z / (4d) exactly (the scalings by
// 4 are exact there), the divisions are corrected reciprocal products and the
// per-scale (4d, 1/(4d)) pairs come from a 128-entry table in LDS.
// Otherwise every division is a true binary32 division.
template <bool ROTATE, bool FAST>
__device__ __forceinline__ void encode_block(float lo[8], float hi[8], float g, float rg,
                                             const float2* __restrict__ tab, uint32_t* sb_out,
                                             u32x2* w_out) {
  if (ROTATE) {
    stages_1_2_4(lo);
    stages_1_2_4(hi);
    stage_8(lo, hi);
  }
  float az = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    az = __builtin_fmaxf(__builtin_fmaxf(az, __builtin_fabsf(lo[i])), __builtin_fabsf(hi[i]));
  uint32_t sb;
  if (FAST) {
    const float ab = ROTATE ? 0.25f * az : az;
    const float a6 = div_corrected(ab, 6.0f, kRecip6);
    // A quotient too large for binary32 makes the product NaN; fminf keeps
    // 448, the right byte for any block value that large.
    sb = e4m3_byte(div_corrected(a6, g, rg));
    const float2 t = tab[sb];
    if (az <= kQuotientLimit * t.x) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lo[i] = div_corrected(lo[i], t.x, t.y);
        hi[i] = div_corrected(hi[i], t.x, t.y);
      }
    } else {
      // Only with a global scale from elsewhere (the amax of an earlier
      // step) can a block's quotients approach the binary32 range; divide
      // exactly (y = z / 4 and d = 4d / 4 are exact here).
      const float d = ROTATE ? 0.25f * t.x : t.x;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lo[i] = (ROTATE ? 0.25f * lo[i] : lo[i]) / d + 0.0f;
        hi[i] = (ROTATE ? 0.25f * hi[i] : hi[i]) / d + 0.0f;
      }
    }
  } else {
    if (ROTATE) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lo[i] = 0.25f * lo[i];
        hi[i] = 0.25f * hi[i];
      }
    }
    const float ab = ROTATE ? 0.25f * az : az;
    sb = e4m3_byte((ab / 6.0f) / g);
    const float sf = e4m3_value(sb) * g;
    const float d = sf == 0.0f ? 1.0f : sf;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lo[i] = lo[i] / d + 0.0f;
      hi[i] = hi[i] / d + 0.0f;
    }
  }
  *sb_out = sb;
  *w_out = u32x2{e2m1_pack8(lo), e2m1_pack8(hi)};
}

// Pass 2 over row-major chunks (256 consecutive blocks, a block per lane).
// Workgroup w handles the chunks w, w + G, w + 2G, ... (G = grid size), last
// chunk first: the chunks pass 1 read last are the likeliest to still be in
// the last-level cache.  The first chunk's blocks were loaded before the
// prologue, so its iteration is peeled off.
template <typename T, bool ROTATE, bool FAST, bool PRE>
__device__ __forceinline__ void quant_blocks_rm(const T* __restrict__ x, int64_t nb, float g,
                                                const float2* __restrict__ tab,
                                                uint8_t* __restrict__ q, uint8_t* __restrict__ s,
                                                RowMajorScales smap, const HeadGuard& head,
                                                const FirstBlock<T>& first,
                                                const uint4* pre) {
  const int64_t nchunks = smap.chunks(nb);
  const int64_t mine = (nchunks - blockIdx.x + gridDim.x - 1) / gridDim.x;
  const float rg = FAST ? 1.0f / g : 0.0f;
  auto finish = [&](int64_t chunk, float lo[8], float hi[8]) {
    uint32_t sb;
    u32x2 w;
    encode_block<ROTATE, FAST>(lo, hi, g, rg, tab, &sb, &w);
    // Codes are stored non-temporally: nothing reads them back here, and in
    // the last-level cache they would only displace input that this pass
    // re-reads (16384 x 8192: 1.6 us off the step; 32768 x 14336: 4.8 us).
    u32x2* qc = reinterpret_cast<u32x2*>(q) + chunk * kThreads;
    __builtin_nontemporal_store(w, qc + threadIdx.x);
    (s + chunk * kThreads)[threadIdx.x] = static_cast<uint8_t>(sb);
  };
  // With pass 1's maxima in q_out (head.counters set), chunk 0 holds them and
  // chunk 1 the arrival counters: the workgroup that visits chunk 0 waits
  // until every workgroup has counted itself in, writes chunk 0 and then
  // chunk 1; the visitor of chunk 1 skips it.  Both chunks are whole there
  // (the host takes that path from 512 blocks).  head_ok is uniform across
  // the workgroup (wait_for_head synchronizes it).
  auto head_ok = [&](int64_t chunk) -> bool {  // false: skip the chunk
    if (!head.counters || chunk > 1) return true;
    if (chunk == 1) return false;
    wait_for_head(head);
    return true;
  };
  auto head_tail = [&](int64_t chunk) {
    if (head.counters && chunk == 0 && kThreads + threadIdx.x < nb) {
      float lo[8], hi[8];
      load_block(x + kThreads * 16, threadIdx.x, lo, hi);
      finish(1, lo, hi);
    }
  };
  if (mine <= 0) return;
  {
    const int64_t chunk = smap.order((mine - 1) * gridDim.x + blockIdx.x, nchunks);
    if (head_ok(chunk)) {
      if (chunk * kThreads + threadIdx.x < nb) {
        float lo[8], hi[8];
        first.unpack(lo, hi);
        finish(chunk, lo, hi);
      }
      head_tail(chunk);
    }
  }
  int64_t it = mine - 2;
  if (PRE && prefetches_second(mine)) {  // the second chunk, from LDS (see prefetch_second)
    const int64_t chunk = smap.order(it * gridDim.x + blockIdx.x, nchunks);
    if (head_ok(chunk)) {
      if (chunk * kThreads + threadIdx.x < nb) {
        float lo[8], hi[8];
        widen8(pre[threadIdx.x], lo);
        widen8(pre[kThreads + threadIdx.x], hi);
        finish(chunk, lo, hi);
      }
      head_tail(chunk);
    }
    --it;
  }
  for (; it >= 0; --it) {
    const int64_t chunk = smap.order(it * gridDim.x + blockIdx.x, nchunks);
    if (!head_ok(chunk)) continue;
    if (chunk * kThreads + threadIdx.x < nb) {
      float lo[8], hi[8];
      load_block(x + chunk * kThreads * 16, threadIdx.x, lo, hi);
      finish(chunk, lo, hi);
    }
    head_tail(chunk);
  }
}

// Pass 2 over swizzled chunks (see SwizzledScales), in the same order; the
// chunk's scale tiles are assembled in LDS and stored whole.
template <typename T, bool ROTATE, bool FAST, typename SMAP, bool PRE>
__device__ __forceinline__ void quant_blocks(const T* __restrict__ x, int64_t nb, float g,
                                             const float2* __restrict__ tab,
                                             uint8_t* __restrict__ q, uint8_t* __restrict__ s,
                                             SMAP smap, const HeadGuard& head, const uint4* pre) {
  // The swizzled layout never has pass 1's maxima in q_out: the host gives
  // it the amax as one word (its head would span a whole row of tiles).
  (void)head;
  const int64_t nchunks = smap.chunks(nb);
  const int64_t mine = (nchunks - blockIdx.x + gridDim.x - 1) / gridDim.x;
  const float rg = FAST ? 1.0f / g : 0.0f;
  __shared__ uint32_t stage[512];  // 4 scale tiles
  for (int64_t it = mine - 1; it >= 0; --it) {
    const auto tile = smap.split(smap.order(it * gridDim.x + blockIdx.x, nchunks));
    for (uint32_t i = threadIdx.x; i < 512; i += kThreads) stage[i] = 0u;
    __syncthreads();
#pragma unroll 1
    for (int sub = 0; sub < SMAP::kSub; ++sub) {
      int64_t b, si;
      if (!smap.locate(tile, sub, threadIdx.x, &b, &si)) continue;
      float lo[8], hi[8];
      if (PRE && it == mine - 1 && sub == 0) {
        widen8(pre[threadIdx.x], lo);
        widen8(pre[kThreads + threadIdx.x], hi);
      } else {
        load_block(x, b, lo, hi);
      }
      uint32_t sb;
      u32x2 w;
      encode_block<ROTATE, FAST>(lo, hi, g, rg, tab, &sb, &w);
      __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(q + b * 8));
      reinterpret_cast<uint8_t*>(stage)[si] = static_cast<uint8_t>(sb);
    }
    // whole tiles, padding zeros included, in one coalesced store
    __syncthreads();
    int64_t first;
    int ntiles;
    smap.chunk_tiles(tile, &first, &ntiles);
    uint32_t* dst = reinterpret_cast<uint32_t*>(s + first);
    for (uint32_t i = threadIdx.x; i < static_cast<uint32_t>(ntiles) * 128u; i += kThreads)
      dst[i] = stage[i];
    __syncthreads();
  }
}

// amax_src: the amax word (npartials == 0) or pass 1's per-workgroup maxima
// at the head of q (npartials of them, then the arrival counters; amax_out
// receives their maximum).
// Eight workgroups per CU (the grid size assumes it): at most 64 VGPRs.
template <typename T, bool ROTATE, typename SMAP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void rotquant_kernel(
    const T* __restrict__ x, int64_t nb, const uint32_t* amax_src, int npartials,
    float* __restrict__ amax_out, uint32_t spin_limit, int allow_fast, uint8_t* __restrict__ q,
    uint8_t* __restrict__ s, float* __restrict__ gscale_out, SMAP smap) {
  __shared__ float2 tab[128];
  __shared__ uint32_t red[kThreads / 64];
  FirstBlock<T> first;
  if constexpr (!SMAP::kStaged) load_first(x, nb, smap, &first);  // staged: no registers to spare
  constexpr bool kPre = sizeof(T) == 2;
  __shared__ uint4 pre[kPre ? 2 : 1][kPre ? kThreads : 1];  // one element where unused
  if constexpr (kPre) {
    if constexpr (SMAP::kStaged)
      prefetch_first_sw(x, nb, smap, &pre[0][0]);
    else
      prefetch_second(x, nb, smap, &pre[0][0]);
  }
  HeadGuard head{nullptr, 0, spin_limit, gscale_out};
  uint32_t abits;
  if (npartials == 0) {
    abits = *amax_src;
  } else {
    uint32_t m = 0u;
    for (int i = threadIdx.x; i < npartials; i += kThreads) m = umax(m, amax_src[i]);
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    abits = red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) abits = umax(abits, red[i]);
    uint32_t* counters = const_cast<uint32_t*>(amax_src) + kCounterBase;
    // every thread's read of the partials is complete (their values met at
    // the barrier) before the workgroup counts itself in; a relaxed increment
    // needs no cache write-back
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(counters + (blockIdx.x % kCounters) * kCounterStride, 1u,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (blockIdx.x == 0 && threadIdx.x == 0) *amax_out = __uint_as_float(abits);
    head = HeadGuard{counters, gridDim.x, spin_limit, gscale_out};
  }
  const float g = global_scale(__uint_as_float(abits));
  if (blockIdx.x == 0 && threadIdx.x == 0) *gscale_out = g;
  if constexpr (sizeof(T) == 2) {
    // uniform across the grid: every workgroup reads the same amax
    if (allow_fast && abits >= kFastAmaxLo && abits < kFastAmaxHi) {
      if (threadIdx.x < 128) {
        const float sf = e4m3_value(threadIdx.x) * g;
        const float d = (ROTATE ? 4.0f : 1.0f) * (sf == 0.0f ? 1.0f : sf);
        tab[threadIdx.x] = make_float2(d, 1.0f / d);
      }
      __syncthreads();
      if constexpr (SMAP::kStaged)
        quant_blocks<T, ROTATE, true, SMAP, kPre>(x, nb, g, tab, q, s, smap, head, &pre[0][0]);
      else
        quant_blocks_rm<T, ROTATE, true, kPre>(x, nb, g, tab, q, s, smap, head, first, &pre[0][0]);
      return;
    }
  }
  if constexpr (SMAP::kStaged)
    quant_blocks<T, ROTATE, false, SMAP, kPre>(x, nb, g, tab, q, s, smap, head, &pre[0][0]);
  else
    quant_blocks_rm<T, ROTATE, false, kPre>(x, nb, g, tab, q, s, smap, head, first, &pre[0][0]);
}

}  // namespace
}  // namespace nvfp4rq
