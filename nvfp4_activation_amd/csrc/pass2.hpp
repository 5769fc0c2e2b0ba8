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
// (a chunk).  Row-major: 256 consecutive blocks, one per lane.  Swizzled: a
// super-tile of 128 rows x 16 blocks (sub-iterations of 16 lanes per row), so
// that one workgroup writes whole 512-byte scale tiles and whole 128-byte
// lines of codes (lines completed from several L2s are written back
// piecemeal).
// Chunk counts and visit indices are 32-bit (the host keeps the chunk count
// below 2^31), so the loop control stays in scalar registers.
struct RowMajorScales {
  static constexpr bool kStaged = false;
  static constexpr bool kHeadSwap = true;  // the head spans chunks 0 and 1 (see head_order)
  int xcd_order;  // give each XCD runs of 4 consecutive chunks
  int mirror;     // a workgroup per chunk, workgroup i taking chunk nchunks - 1 - i
  __device__ __forceinline__ int64_t operator()(int64_t b) const { return b; }
  __host__ __device__ uint32_t chunks(int64_t nb) const {
    return static_cast<uint32_t>((nb + kThreads - 1) / kThreads);
  }
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
  __host__ __device__ uint32_t order(uint32_t i, uint32_t nchunks) const {
    if (mirror) return nchunks - 1 - i;
    return xcd_order ? (i & ~31u) | ((i & 7u) << 2) | ((i >> 3) & 3u) : i;
  }
};
struct SwizzledScales {
  static constexpr bool kStaged = true;     // scale tiles assembled in LDS
  static constexpr bool kHeadSwap = false;  // the head lies in chunk 0 alone
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
  __host__ __device__ Tile split(uint32_t chunk) const {
    const uint32_t rt = chunk / cs;
    return Tile{rt, chunk - rt * cs};
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
  __host__ __device__ uint32_t chunks(int64_t) const {
    return static_cast<uint32_t>(((rows + 127) / 128) * cs);
  }
  // runs16: visit index i (on XCD i % 8) takes chunk (i & ~127) | ((i & 7)
  // << 4) | ((i >> 3) & 15), so each XCD reads 16 consecutive column windows
  // of a row tile (8 KiB of every bf16 row) instead of one.  Step at
  // 16384 x 8192: 101.5 us against 106.7 in plain order (runs of 2, 4, 8, 32,
  // 64: 122.5, 106.6, 115.4, 101.7, 101.2 us); 4096 x 4096: 22.2 against
  // 23.6 us.  Used when a row tile holds a multiple of 16 windows (at
  // 32768 x 14336, 56 windows, runs of 16 cost 2.7%) and the chunk count is a
  // multiple of 128.
  __host__ __device__ uint32_t order(uint32_t i, uint32_t nchunks) const {
    if (mirror) return nchunks - 1 - i;
    return runs16 ? (i & ~127u) | ((i & 7u) << 4) | ((i >> 3) & 15u) : i;
  }
  // The chunk's tiles (rt, 4 cw .. 4 cw + 3) are consecutive in memory.
  __host__ __device__ void chunk_tiles(Tile t, int64_t* first_byte, int* ntiles) const {
    const int64_t ct0 = static_cast<int64_t>(t.cw) * 4;
    *first_byte = (t.rt * ctiles + ct0) * 512;
    *ntiles = static_cast<int>(ctiles - ct0 < 4 ? ctiles - ct0 : 4);
  }
};

// Number of chunks workgroup wg of a grid of g visits: visit indices wg,
// wg + g, wg + 2g, ... below nchunks.
__host__ __device__ inline uint32_t chunks_of(uint32_t wg, uint32_t g, uint32_t nchunks) {
  return wg < nchunks ? (nchunks - wg + g - 1) / g : 0u;
}

// Launch shape of the quantize pass, computed once on the host and passed as
// one argument, so that a workgroup's first addresses and its fast-path
// decision need nothing read later: the chunk count, the grid size, and the
// number of chunks each workgroup visits from nchunks = base * grid + extra
// (a division on the device would be emulated on the vector unit and delay
// each workgroup's first loads): base + 1 for wg < extra, base for the
// others.  allow_fast: 0 forces the exact divisions (tests).
struct Launch {
  uint32_t nchunks, base, extra, grid;
  int allow_fast;
  __host__ __device__ uint32_t of(uint32_t wg) const { return base + (wg < extra ? 1u : 0u); }
  __host__ static Launch make(uint32_t nchunks, uint32_t grid, int allow_fast = 1) {
    return Launch{nchunks, nchunks / grid, nchunks % grid, grid, allow_fast};
  }
};

// Where the quantize pass takes the global amax from (a template argument,
// so that each workgroup's first loads depend on nothing read at run time):
//   kHead   pass 1's per-workgroup maxima at the head of an output (below);
//   kWord   one amax word written by pass 1 on the same tensor;
//   kGiven  one amax word kept from elsewhere (the given-scale call): block
//           quotients may then leave the range the fast quotient is proven
//           on, and such blocks divide exactly.
enum AmaxMode { kHead = 0, kWord = 1, kGiven = 2 };

// ---------------------------------------------------------------- head of the output

// When pass 1 leaves its per-workgroup maxima at the head of the outputs,
// every pass-2 workgroup reads them in its prologue and then counts itself in
// on one of the arrival counters.  Row-major scales: the head is the first
// 4 KiB of the codes, chunk 0's bytes (the maxima) and chunk 1's (the
// counters).  Workgroup 0 alone writes both chunks: the visit order is changed
// so that its last two visits are chunk 1 (visit G, G the grid size) and then
// chunk 0 (visit 0); the workgroup that the plain order gives chunk 1 takes
// chunk order(G) instead, so every workgroup keeps its number of chunks (the
// host launches at most nchunks - 1 workgroups, so that workgroup 0 has both
// visits).  Before storing chunk 1 it waits for every workgroup to have
// counted itself in.  Swizzled scales: the maxima fill chunk 0's scale tiles
// and the counters sit in chunk 0's code rows, so workgroup 0's last visit,
// chunk 0 in the plain order, is the whole head and needs no swap; it waits
// before storing any of it.  Nobody else waits, so the count always
// completes, and no counter is written over while another workgroup still
// reads it.  Chunks run last-first, so that wait comes after all of
// workgroup 0's other chunks.  It is bounded in time: past `ticks` of the
// device's constant-rate wall clock the workgroup goes on and marks the call
// failed with a NaN global scale and a NaN amax (the codes and scales are
// then unspecified).
template <typename SMAP>
__host__ __device__ inline uint32_t head_order(const SMAP& smap, uint32_t i, uint32_t nchunks, uint32_t grid,
                                               bool head) {
  if (!head || !SMAP::kHeadSwap) return smap.order(i, nchunks);
  if (i == grid) return 1u;
  const uint32_t c = smap.order(i, nchunks);
  return c == 1u ? smap.order(grid, nchunks) : c;
}

struct HeadGuard {
  Counters counters;   // base null: the amax came as one word
  uint32_t need;       // quantize workgroups
  uint64_t ticks;
  float* gscale_out;
  float* amax_out;
};

__device__ __forceinline__ void wait_for_head(const HeadGuard& h) {
  __shared__ int timed_out;
  if (threadIdx.x < 64) {  // wave 0: one counter per lane of its first row (lanes past kCounters add 0)
    const uint64_t t0 = static_cast<uint64_t>(wall_clock64());
    int late = 0;
    // Each poll reads a counter with a fetch-and-add of zero: an atomic,
    // performed where the increments are performed, so no copy of the line
    // in another cache can answer it.  Relaxed ordering: acquire/release at
    // agent scope would write back or invalidate the L2 of every XCD
    // involved on each poll.  Nothing written by other workgroups is read
    // after the wait; the waiter's stores follow the loop.
    // The compiler turns an add of a literal 0 back into a load, so the zero
    // is made opaque to it (an empty asm statement that only claims to
    // change the register).
    uint32_t zero = 0u;
    __asm__ volatile("" : "+v"(zero));
    for (;;) {
      static_assert(kCounters == 16, "the counters fill the wave's first row");
      const uint32_t c = threadIdx.x < kCounters
                             ? __hip_atomic_fetch_add(h.counters.at(threadIdx.x), zero, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT)
                             : 0u;
      if (row0_sum_u32(c) >= h.need) break;
      if (static_cast<uint64_t>(wall_clock64()) - t0 > h.ticks) {
        late = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (threadIdx.x == 0) timed_out = late;
  }
  __syncthreads();
  if (timed_out && threadIdx.x == 0) {
    *h.gscale_out = __uint_as_float(0x7FC00000u);
    if (h.amax_out) *h.amax_out = __uint_as_float(0x7FC00000u);
  }
}

// ---------------------------------------------------------------- raw buffer access

// Row-major chunks are read and written through raw buffer resources whose
// base is the chunk's first byte and whose size is its valid part: the
// address arithmetic stays in scalar registers, and in the tensor's last,
// partial chunk the lanes past its end load zeros and have their stores
// dropped by the hardware's range check, so no lane needs a bounds test.

// A lane's block as raw bits.
template <typename T>
struct Block;
template <>
struct Block<uint16_t> {
  u32x4 a, b;
  __device__ __forceinline__ void load(const uint16_t* x, uint32_t chunk, uint32_t valid, uint32_t tid) {
    const auto r = chunk_rsrc(x + static_cast<int64_t>(chunk) * (kThreads * 16), valid * 32u);
    a = __builtin_amdgcn_raw_buffer_load_b128(r, tid * 32u, 0, 0);
    b = __builtin_amdgcn_raw_buffer_load_b128(r, tid * 32u + 16u, 0, 0);
  }
  // block `blk` of a buffer resource that starts at a block boundary
  __device__ __forceinline__ void load_at(__amdgpu_buffer_rsrc_t r, uint32_t blk) {
    a = __builtin_amdgcn_raw_buffer_load_b128(r, blk * 32u, 0, 0);
    b = __builtin_amdgcn_raw_buffer_load_b128(r, blk * 32u + 16u, 0, 0);
  }
  __device__ __forceinline__ void unpack(float lo[8], float hi[8]) const {
    widen8(make_uint4(a.x, a.y, a.z, a.w), lo);
    widen8(make_uint4(b.x, b.y, b.z, b.w), hi);
  }
};
template <>
struct Block<float> {
  u32x4 a, b, c, d;
  __device__ __forceinline__ void load(const float* x, uint32_t chunk, uint32_t valid, uint32_t tid) {
    const auto r = chunk_rsrc(x + static_cast<int64_t>(chunk) * (kThreads * 16), valid * 64u);
    a = __builtin_amdgcn_raw_buffer_load_b128(r, tid * 64u, 0, 0);
    b = __builtin_amdgcn_raw_buffer_load_b128(r, tid * 64u + 16u, 0, 0);
    c = __builtin_amdgcn_raw_buffer_load_b128(r, tid * 64u + 32u, 0, 0);
    d = __builtin_amdgcn_raw_buffer_load_b128(r, tid * 64u + 48u, 0, 0);
  }
  __device__ __forceinline__ void load_at(__amdgpu_buffer_rsrc_t r, uint32_t blk) {
    a = __builtin_amdgcn_raw_buffer_load_b128(r, blk * 64u, 0, 0);
    b = __builtin_amdgcn_raw_buffer_load_b128(r, blk * 64u + 16u, 0, 0);
    c = __builtin_amdgcn_raw_buffer_load_b128(r, blk * 64u + 32u, 0, 0);
    d = __builtin_amdgcn_raw_buffer_load_b128(r, blk * 64u + 48u, 0, 0);
  }
  __device__ __forceinline__ void unpack(float lo[8], float hi[8]) const {
    const u32x4 v[4] = {a, b, c, d};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float* o = k < 2 ? lo + 4 * k : hi + 4 * (k - 2);
      o[0] = __uint_as_float(v[k].x);
      o[1] = __uint_as_float(v[k].y);
      o[2] = __uint_as_float(v[k].z);
      o[3] = __uint_as_float(v[k].w);
    }
  }
};

// Codes (8 bytes per lane, stored non-temporally: nothing reads them back
// here, and in the last-level cache they would only displace input that this
// pass re-reads: 16384 x 8192 step 1.6 us faster, 32768 x 14336 4.8 us) and
// the scale byte (the low byte of sb) of chunk `chunk`.
__device__ __forceinline__ void store_chunk_block(uint8_t* q, uint8_t* s, uint32_t chunk, uint32_t valid,
                                                  uint32_t tid, u32x2 w, uint32_t sb) {
  const auto rq = chunk_rsrc(q + static_cast<int64_t>(chunk) * (kThreads * 8), valid * 8u);
  __builtin_amdgcn_raw_buffer_store_b64(w, rq, tid * 8u, 0, kNontemporal);
  const auto rs = chunk_rsrc(s + static_cast<int64_t>(chunk) * kThreads, valid);
  __builtin_amdgcn_raw_buffer_store_b8(static_cast<unsigned char>(sb), rs, tid, 0, 0);
}

// The lane's block of the workgroup's second chunk (bf16, row-major), loaded
// before the prologue straight into LDS (the kernel has no registers to spare
// for it), 8 KiB per workgroup: 16384 x 8192 step 97.5 -> 95.7 us, pass 2
// 52.6 -> 51.1 us (three A/B pairs).  Through a buffer resource whose size is
// the chunk's valid part (0 when the workgroup has fewer than two chunks), so
// the loads are issued unconditionally: with no branch between wave 0's loads
// of the maxima and their use, the wait for them can leave these loads in
// flight.  quant_blocks_rm reads the block back when prefetches_second.
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;
__device__ __forceinline__ bool prefetches_second(uint32_t mine) { return mine >= 2; }
__device__ __forceinline__ void prefetch_second(const uint16_t* __restrict__ x, int64_t nb,
                                                RowMajorScales smap, Launch vis, bool head, uint4* pre) {
  const uint32_t nchunks = vis.nchunks;
  const uint32_t mine = vis.of(blockIdx.x);
  const bool on = prefetches_second(mine);
  const uint32_t c = on ? head_order(smap, (mine - 2) * vis.grid + blockIdx.x, nchunks, vis.grid, head) : 0u;
  const uint32_t nfull = static_cast<uint32_t>(nb / kThreads);
  const uint32_t valid = !on ? 0u : c < nfull ? static_cast<uint32_t>(kThreads) : static_cast<uint32_t>(nb % kThreads);
  const auto r = chunk_rsrc(x + static_cast<int64_t>(c) * (kThreads * 16), valid * 32u);
  // pre holds the blocks' first halves at [0, kThreads) and their second
  // halves at [kThreads, 2 kThreads).  The destination is per wave: lane l's
  // 16 bytes land at slot 64 w + l, i.e. at threadIdx.x.  Address-space
  // conversions take C-style casts.
  const int w = threadIdx.x >> 6;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)(pre + w * 64), 16, threadIdx.x * 32u, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)(pre + kThreads + w * 64), 16,
                                           threadIdx.x * 32u + 16u, 0, 0, 0);
}

// Swizzled chunks: the lane's block of the first sub-iteration of the
// workgroup's first chunk, loaded into LDS before the prologue (the pass has
// no registers to spare for the row-major pass's early first-block load):
// 16384 x 8192 swizzled step 101.3 -> 100.65 us, three A/B pairs.
template <int NT>
__device__ __forceinline__ void prefetch_first_sw(const uint16_t* __restrict__ x, int64_t nb,
                                                  SwizzledScales smap, Launch vis, bool head, uint4* pre) {
  (void)nb;
  // Through a buffer resource over the chunk's row tile (its size 0 when the
  // workgroup has no chunk; lanes outside the tensor get an offset past the
  // end), so the loads are issued unconditionally, as in prefetch_second.
  const uint32_t nchunks = vis.nchunks;
  const uint32_t mine = vis.of(blockIdx.x);
  const auto tile =
      smap.split(mine > 0 ? head_order(smap, (mine - 1) * vis.grid + blockIdx.x, nchunks, vis.grid, head) : 0u);
  const int64_t row0 = tile.rt * 128;
  const uint32_t rows_here =
      mine == 0 ? 0u : static_cast<uint32_t>(smap.rows - row0 < 128 ? smap.rows - row0 : 128);
  const auto r = chunk_rsrc(x + row0 * smap.cb * 16, rows_here * smap.cb * 32u);
  const uint32_t rr = threadIdx.x >> 4, c = tile.cw * 16 + (threadIdx.x & 15u);
  const uint32_t off = rr < rows_here && c < smap.cb ? (rr * smap.cb + c) * 32u : 0xFFFFFFE0u;
  const int w = threadIdx.x >> 6;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)(pre + w * 64), 16, off, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)(pre + NT + w * 64), 16, off + 16u, 0, 0, 0);
}

// ---------------------------------------------------------------- one block

// One block of pass 2, in one lane: rotation (in place on lo, hi), the block
// scale byte and the two words of E2M1 codes.  Every step is the definition
// of section 2 (hadamard_nvfp4_kernel) in binary32:
//   z     = S16 x                         (butterfly, no scaling yet)
//   a_b   = max |y| = 0.25 max |z|        (exact for any rounding, see pass 1)
//   v     = (a_b / 6) / g,  s = E4M3(min(v, 448))
//   d     = float(s) * g, or 1 when that is 0
//   code  = E2M1(y / d),  y = 0.25 z
// FAST (bf16 in the guarded range): the scalings by 4 are exact there, so
// a_b / 6 = max |z| / 24 and y / d = z / (4d); the block value's divisions are
// corrected reciprocal products, and each element's code comes from the
// two-word reciprocal of 4d (a 128-entry LDS table indexed by the scale
// byte).  Otherwise every division is a true binary32 division.  GUARD: the
// global scale may come from another tensor's amax, so a block's quotients
// can exceed the range the two-word quotient is proven on; such a block
// divides exactly.  sb_out: the scale byte in bits 0..7, other bits
// unspecified.
// The first half: z = S16 x in place (x itself when not rotating) and the
// block's largest |z|.  Needs no scale, so a workgroup's first block goes
// through it while the prologue derives the scales.
template <bool ROTATE>
__device__ __forceinline__ float rotate_block(float lo[8], float hi[8]) {
  if (ROTATE) {
    stages_1_2_4(lo);
    stages_1_2_4(hi);
    stage_8(lo, hi);
  }
  float az = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    az = __builtin_fmaxf(__builtin_fmaxf(az, __builtin_fabsf(lo[i])), __builtin_fabsf(hi[i]));
  return az;
}

// The second half, from rotate_block's output.
template <bool ROTATE, bool FAST, bool GUARD>
__device__ __forceinline__ void quantize_block(float lo[8], float hi[8], float az, float g, float rg,
                                               const float2* __restrict__ tab, uint32_t* sb_out,
                                               u32x2* w_out) {
  uint32_t sb;
  if (FAST) {
    const float a6 = ROTATE ? div_corrected(az, 24.0f, kRecip24) : div_corrected(az, 6.0f, kRecip6);
    // A quotient too large for binary32 makes the product NaN; fminf keeps
    // 448, the right byte for any block value that large.
    sb = e4m3_byte_lo(div_corrected(a6, g, rg));
    const float2 t = tab[sb & 0xFFu];
    if (!GUARD || az * t.x <= kQuotientLimit) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lo[i] = quot2(lo[i], t.x, t.y);
        hi[i] = quot2(hi[i], t.x, t.y);
      }
    } else {
      // Only with a global scale from elsewhere (the amax of an earlier
      // step) can a block's quotients approach the binary32 range; divide
      // exactly (y = z / 4 is exact here).
      const float sf = e4m3_value(sb & 0xFFu) * g;
      const float d = sf == 0.0f ? 1.0f : sf;
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

template <bool ROTATE, bool FAST, bool GUARD>
__device__ __forceinline__ void encode_block(float lo[8], float hi[8], float g, float rg,
                                             const float2* __restrict__ tab, uint32_t* sb_out,
                                             u32x2* w_out) {
  const float az = rotate_block<ROTATE>(lo, hi);
  quantize_block<ROTATE, FAST, GUARD>(lo, hi, az, g, rg, tab, sb_out, w_out);
}

// ---------------------------------------------------------------- chunk loops

// Pass 2 over row-major chunks (256 consecutive blocks, a block per lane).
// Workgroup w handles the chunks of visits w, w + G, w + 2G, ... (G = grid
// size), last visit first: the chunks pass 1 read last are the likeliest to
// still be in the last-level cache.  The first chunk's blocks were loaded
// before the prologue, so its iteration is peeled off.
template <typename T, bool ROTATE, bool FAST, bool GUARD, bool PRE>
__device__ __forceinline__ void quant_blocks_rm(const T* __restrict__ x, int64_t nb, float g, float rg,
                                                const float2* __restrict__ tab, uint8_t* q, uint8_t* s,
                                                RowMajorScales smap, Launch vis, const HeadGuard& head,
                                                float flo[8], float fhi[8], float faz, const uint4* pre) {
  const uint32_t nchunks = vis.nchunks;
  const uint32_t nfull = static_cast<uint32_t>(nb / kThreads);
  const uint32_t tail = static_cast<uint32_t>(nb % kThreads);
  const uint32_t grid = vis.grid, wg = blockIdx.x, tid = threadIdx.x;
  const uint32_t mine = vis.of(wg);
  auto valid = [&](uint32_t chunk) -> uint32_t { return chunk < nfull ? kThreads : tail; };
  const bool hd = head.counters.base != nullptr;
  auto store = [&](uint32_t chunk, u32x2 w, uint32_t sb) {
    // chunk 1 holds the arrival counters: its writer (workgroup 0, see
    // head_order) waits for the full count first; chunk 0 comes after it.
    // Uniform across the workgroup (wait_for_head synchronizes it).
    if (hd && chunk == 1) wait_for_head(head);
    store_chunk_block(q, s, chunk, valid(chunk), tid, w, sb);
  };
  auto finish = [&](uint32_t chunk, float lo[8], float hi[8]) {
    uint32_t sb;
    u32x2 w;
    encode_block<ROTATE, FAST, GUARD>(lo, hi, g, rg, tab, &sb, &w);
    store(chunk, w, sb);
  };
  auto visit = [&](int32_t it) { return head_order(smap, static_cast<uint32_t>(it) * grid + wg, nchunks, grid, hd); };
  if (mine == 0) return;
  {  // the first chunk's block, rotated before the prologue's barrier
    uint32_t sb;
    u32x2 w;
    quantize_block<ROTATE, FAST, GUARD>(flo, fhi, faz, g, rg, tab, &sb, &w);
    store(visit(static_cast<int32_t>(mine) - 1), w, sb);
  }
  int32_t it = static_cast<int32_t>(mine) - 2;  // mine < 2^31
  if (PRE && prefetches_second(mine)) {  // the second chunk, from LDS (see prefetch_second)
    float lo[8], hi[8];
    widen8(pre[tid], lo);
    widen8(pre[kThreads + tid], hi);
    finish(visit(it), lo, hi);
    --it;
  }
  for (; it >= 0; --it) {
    const uint32_t chunk = visit(it);
    Block<T> blk;
    blk.load(x, chunk, valid(chunk), tid);
    float lo[8], hi[8];
    blk.unpack(lo, hi);
    finish(chunk, lo, hi);
  }
}

// Pass 2 over swizzled chunks (see SwizzledScales), in the same order; the
// chunk's scale tiles are assembled in LDS and stored whole, and its codes
// are stored as they are computed.  With pass 1's maxima at the head
// (head.counters set), chunk 0 holds the maxima in its scale tiles and the
// arrival counters in its first code rows; workgroup 0, whose last visit it
// is, waits before starting it.
template <typename T, bool ROTATE, bool FAST, typename SMAP, bool PRE, int NT>
__device__ __forceinline__ void quant_blocks(const T* __restrict__ x, int64_t nb, float g, float rg,
                                             const float2* __restrict__ tab, uint8_t* q, uint8_t* s,
                                             SMAP smap, Launch vis, const HeadGuard& head, const uint4* pre) {
  const uint32_t nchunks = vis.nchunks;
  const uint32_t mine = vis.of(blockIdx.x);
  const bool hd = head.counters.base != nullptr;
  __shared__ uint32_t stage[512];  // 4 scale tiles
  for (int32_t it = static_cast<int32_t>(mine) - 1; it >= 0; --it) {
    const uint32_t chunk =
        head_order(smap, static_cast<uint32_t>(it) * vis.grid + blockIdx.x, nchunks, vis.grid, hd);
    // chunk 0 is the head (its scale tiles hold the maxima, its first code
    // rows the counters): its writer, workgroup 0, waits before any store.
    // Uniform across the workgroup (wait_for_head synchronizes it).
    if (hd && chunk == 0) wait_for_head(head);
    const auto tile = smap.split(chunk);
    // The chunk's row tile through raw buffer resources (block offsets within
    // the tile fit in 32 bits: the host keeps 128 rows of input below 2^31
    // bytes); the prefetched first blocks come from LDS.
    const int64_t row0 = tile.rt * 128;
    const uint32_t rows_here = static_cast<uint32_t>(smap.rows - row0 < 128 ? smap.rows - row0 : 128);
    const int64_t tile_blocks = row0 * smap.cb;
    const auto rx = chunk_rsrc(x + tile_blocks * 16, rows_here * smap.cb * 16u * static_cast<uint32_t>(sizeof(T)));
    const auto rq = chunk_rsrc(q + tile_blocks * 8, rows_here * smap.cb * 8u);
    for (uint32_t i = threadIdx.x; i < 512; i += NT) stage[i] = 0u;
    __syncthreads();
    const uint32_t c = tile.cw * 16 + (threadIdx.x & 15u);
    // NT / 16 rows of 16 blocks per sub-iteration
    constexpr int kSubs = 128 / (NT / 16);
#pragma unroll 1
    for (int sub = 0; sub < kSubs; ++sub) {
      const uint32_t r = static_cast<uint32_t>(sub) * (NT / 16) + (threadIdx.x >> 4);  // row within the tile
      if (r >= rows_here || c >= smap.cb) continue;
      const uint32_t blk = r * smap.cb + c;
      float lo[8], hi[8];
      if (PRE && it == static_cast<int32_t>(mine) - 1 && sub == 0) {
        widen8(pre[threadIdx.x], lo);
        widen8(pre[NT + threadIdx.x], hi);
      } else {
        Block<T> bl;
        bl.load_at(rx, blk);
        bl.unpack(lo, hi);
      }
      uint32_t sb;
      u32x2 w;
      encode_block<ROTATE, FAST, false>(lo, hi, g, rg, tab, &sb, &w);
      __builtin_amdgcn_raw_buffer_store_b64(w, rq, blk * 8u, 0, kNontemporal);
      reinterpret_cast<uint8_t*>(stage)[SwizzledScales::place(r, c & 15u, 4)] = static_cast<uint8_t>(sb);
    }
    __syncthreads();
    // whole tiles, padding zeros included, in one coalesced store
    int64_t first;
    int ntiles;
    smap.chunk_tiles(tile, &first, &ntiles);
    uint32_t* dst = reinterpret_cast<uint32_t*>(s + first);
    for (uint32_t i = threadIdx.x; i < static_cast<uint32_t>(ntiles) * 128u; i += NT)
      dst[i] = stage[i];
    __syncthreads();
  }
}

// ---------------------------------------------------------------- kernel

// amax_src: the amax word (kWord, kGiven) or pass 1's per-workgroup maxima
// at the head of q (row-major) or s (swizzled): kMaxPartials words, those
// past pass 1's grid cleared, with the arrival counters at `counters`;
// amax_out receives their maximum.  q and s carry no
// __restrict__: the head is read and counted on through amax_src and later
// overwritten through q or s.
// Eight waves per SIMD (the grid size assumes it): at most 64 VGPRs.  NT: the
// workgroup size, kThreads, or for swizzled scales also 1024 (small tensors:
// a chunk's 128 rows in 2 sub-iterations instead of 8).
template <typename T, bool ROTATE, typename SMAP, AmaxMode MODE, int NT = kThreads>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8))) void rotquant_kernel(
    const T* __restrict__ x, int64_t nb, uint32_t* amax_src, Counters counters, float* amax_out,
    uint64_t head_ticks, uint8_t* q, uint8_t* s, float* gscale_out, SMAP smap, Launch vis) {
  constexpr bool hd = MODE == kHead;
  constexpr bool kGuard = MODE == kGiven;
  static_assert(NT == kThreads || (SMAP::kStaged && NT == 1024), "workgroup size");
  __shared__ float2 tab[128];
  // pass 1's maxima (kMaxPartials words in the head's first 2 KiB, those
  // past its grid cleared by pass 1: two 16-byte loads per lane) are loaded
  // first, by every wave although only wave 0 reduces them: with no branch
  // between these loads and their use, wave 0's wait for them leaves the
  // block loads and the LDS prefetch below in flight (loads complete in
  // issue order).
  u32x4 part0 = {0u, 0u, 0u, 0u}, part1 = {0u, 0u, 0u, 0u};
  if constexpr (hd) {
    const u32x4* p4 = reinterpret_cast<const u32x4*>(amax_src);
    part0 = p4[threadIdx.x & 63u];
    part1 = p4[64 + (threadIdx.x & 63u)];
  }
  // The first chunk's block, through a buffer resource of the chunk's valid
  // size (0 when the workgroup has no chunk): unconditional, as above.
  Block<T> first;
  if constexpr (!SMAP::kStaged) {  // staged: no registers to spare
    const uint32_t mine = vis.of(blockIdx.x);
    const uint32_t nfull = static_cast<uint32_t>(nb / kThreads);
    const uint32_t c =
        mine > 0 ? head_order(smap, (mine - 1) * vis.grid + blockIdx.x, vis.nchunks, vis.grid, hd) : 0u;
    const uint32_t valid =
        mine == 0 ? 0u : c < nfull ? static_cast<uint32_t>(kThreads) : static_cast<uint32_t>(nb % kThreads);
    first.load(x, c, valid, threadIdx.x);
  }
  constexpr bool kPre = sizeof(T) == 2;
  __shared__ uint4 pre[kPre ? 2 : 1][kPre ? NT : 1];  // one element where unused
  if constexpr (kPre) {
    if constexpr (SMAP::kStaged)
      prefetch_first_sw<NT>(x, nb, smap, vis, hd, &pre[0][0]);
    else
      prefetch_second(x, nb, smap, vis, hd, &pre[0][0]);
  }
  // Prologue.  Wave 0 alone derives the scalars: the global amax (pass 1's
  // maxima reduced across the wave, then counted in, or the word), g =
  // (A / 6) / 448 and, on the fast path, 1/g and the 128 two-word reciprocals
  // (two entries per lane; entry 0, a constant, leaves lane 0's first slot
  // to 1/g, through the same correctly rounded division); meanwhile every
  // wave rotates its first block, which needs no scale.  One barrier then
  // hands the scalars to all waves.  (Deriving them in every wave instead,
  // each with a quarter of the table: 4096 x 4096 pass 2 8.0 against 7.7 us;
  // the waves' extra work costs more than the shorter chain saves.)
  __shared__ uint32_t sh_abits;
  __shared__ float sh_g, sh_rg;
  if (threadIdx.x < 64) {
    uint32_t abits;
    if constexpr (hd) {
      // the words past pass 1's grid were cleared by pass 1: no mask
      const uint32_t m = umax(umax(umax(part0.x, part0.y), umax(part0.z, part0.w)),
                              umax(umax(part1.x, part1.y), umax(part1.z, part1.w)));
      abits = wave_max_u32_uniform(m);
      // this workgroup's reads of the maxima are complete (their values met
      // in the reduction) before it counts itself in; a relaxed increment
      // needs no cache write-back
      if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(counters.at(blockIdx.x % kCounters), 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        if (blockIdx.x == 0) *amax_out = __uint_as_float(abits);
      }
    } else {
      abits = *amax_src;
    }
    float g, rg = 0.0f;
    if (sizeof(T) == 2 && vis.allow_fast && abits >= kFastAmaxLo && abits < kFastAmaxHi) {
      g = global_scale_corrected(__uint_as_float(abits));
      // entry k: D = 4 E4M3(k) g (rotated input; E4M3(k) g unrotated), never
      // zero in this range except for k = 0, whose D is then 4 (or 1) and
      // whose reciprocal is exactly (1/4, 0) (or (1, 0))
      constexpr float kUnit = ROTATE ? 4.0f : 1.0f;
      const uint32_t k0 = threadIdx.x, k1 = threadIdx.x + 64;
      const float2 r0 = recip2_corrected(k0 == 0 ? g : kUnit * (e4m3_value(k0) * g));
      const float2 r1 = recip2_corrected(kUnit * (e4m3_value(k1) * g));
      rg = r0.x;  // lane 0's
      tab[k0] = k0 == 0 ? make_float2(1.0f / kUnit, 0.0f) : r0;
      tab[k1] = r1;
    } else {
      g = global_scale(__uint_as_float(abits));
    }
    if (threadIdx.x == 0) {
      sh_abits = abits;
      sh_g = g;
      sh_rg = rg;
      if (blockIdx.x == 0) *gscale_out = g;
    }
  }
  float flo[8], fhi[8], faz = 0.0f;
  if constexpr (!SMAP::kStaged) {
    first.unpack(flo, fhi);
    faz = rotate_block<ROTATE>(flo, fhi);
  }
  __syncthreads();
  const uint32_t abits = sh_abits;
  const float g = sh_g, rg = sh_rg;
  const HeadGuard head{hd ? counters : Counters{nullptr, 0u}, vis.grid, head_ticks, gscale_out, amax_out};
  if constexpr (sizeof(T) == 2) {
    // uniform across the grid: every workgroup reads the same amax
    if (vis.allow_fast && abits >= kFastAmaxLo && abits < kFastAmaxHi) {
      if constexpr (SMAP::kStaged)
        quant_blocks<T, ROTATE, true, SMAP, kPre, NT>(x, nb, g, rg, tab, q, s, smap, vis, head, &pre[0][0]);
      else
        quant_blocks_rm<T, ROTATE, true, kGuard, kPre>(x, nb, g, rg, tab, q, s, smap, vis, head, flo, fhi, faz,
                                                      &pre[0][0]);
      return;
    }
  }
  if constexpr (SMAP::kStaged)
    quant_blocks<T, ROTATE, false, SMAP, kPre, NT>(x, nb, g, rg, tab, q, s, smap, vis, head, &pre[0][0]);
  else
    quant_blocks_rm<T, ROTATE, false, kGuard, kPre>(x, nb, g, rg, tab, q, s, smap, vis, head, flo, fhi, faz,
                                                   &pre[0][0]);
}

}  // namespace
}  // namespace nvfp4rq
