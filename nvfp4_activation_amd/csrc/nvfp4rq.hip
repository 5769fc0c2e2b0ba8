// Fused block-Hadamard rotation + NVFP4 activation quantization for gfx950.
//
// Method: page "A Fused Hadamard + NVFP4 Quantization Kernel in Triton"
// (kanthi.in), sections 1-3; stored layout: page "NVFP4 Quantization"
// (atlas-docs), section "The numeric format".  The C ABI and its contract are
// in include/nvfp4rq.h.
//
// Two passes over the input:
//   rotamax   reads every 16-value block, rotates it in registers, and keeps
//             the running max |y| as binary32 bits (non-negative floats order
//             like unsigned integers, so the max is exact and independent of
//             the reduction order); wave and workgroup maxima, then one
//             atomicMax per workgroup into the caller's amax word.
//   rotquant  every workgroup derives the global scale from that word, then
//             each lane loads a block, rotates it, scales and encodes it, and
//             writes 8 code bytes and 1 scale byte.  The rotated tensor never
//             leaves registers.
//
// Arithmetic: binary32, round to nearest even, denormals kept (gfx950
// default), no contraction (-ffp-contract=off); the divisions are the
// compiler's correctly rounded binary32 division.

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdlib>
#include <cstdint>
#include <tuple>
#include <utility>

#include "nvfp4rq.h"
#include "nvfp4rq_device.hpp"

namespace {

using namespace nvfp4rq;

constexpr int kThreads = 256;      // 4 waves of 64
constexpr int kAmaxPieces = 8;     // 16-byte pieces per lane per iteration in the bf16 amax pass

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
constexpr int64_t kLastLevelKeep = 176LL << 20;  // bytes of input pass 1 leaves cached
// Arrival counters of the quantize pass when pass 1 leaves its partial maxima
// in q_out: spread over kCounters words on separate 128-byte lines, since
// thousands of increments of one word serialize (and a workgroup's loads
// wait behind its own pending atomic).
constexpr int kCounters = 64;
constexpr int kCounterStride = 32;  // words
__host__ __device__ constexpr int64_t counter_base(int64_t npartials) {
  return (npartials + kCounterStride - 1) / kCounterStride * kCounterStride;  // words
}
__host__ __device__ constexpr int64_t head_bytes(int64_t npartials) {
  return 4 * (counter_base(npartials) + kCounters * kCounterStride);
}

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t u) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
    u = umax(u, static_cast<uint32_t>(__shfl_xor(static_cast<int>(u), off, 64)));
  return u;
}

// Workgroup maximum, then either one atomicMax per workgroup on a zeroed word
// (partials == 0), or a plain store of the workgroup's maximum to out[wg]
// (partials == 1; workgroup 0 also clears the arrival counters the quantize
// pass uses, so no word has to be zeroed beforehand).  Non-negative binary32
// values order like their bit patterns, so the maximum is exact and the same
// for any reduction order (a NaN input stays visible as bits above +inf).
__device__ __forceinline__ void workgroup_max_to(uint32_t m, uint32_t* __restrict__ out,
                                                 int partials) {
  __shared__ uint32_t part[kThreads / 64];
  m = wave_max_u32(m);
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
  if (partials && blockIdx.x == 0 && threadIdx.x < kCounters)
    out[counter_base(gridDim.x) + threadIdx.x * kCounterStride] = 0u;
}

__device__ __forceinline__ uint32_t abs_bits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// ---------------------------------------------------------------- kernels

__global__ void zero_word_kernel(uint32_t* __restrict__ w) { *w = 0u; }

// Pass 1 for bf16 (section 2: the global scale needs the amax of the whole
// rotated tensor before any block can be scaled).  Coalesced: in each
// iteration a wave reads 64 * kAmaxPieces consecutive 16-byte pieces, lane l
// taking pieces l, l + 64, ...; a piece is half a block, so lanes 2k and 2k+1
// hold elements 0..7 and 8..15 of one block.  Each lane runs the stride-1, 2,
// 4 stages on its half; the stride-8 stage pairs the two lanes, and
// max(|a + b|, |a - b|) = RN(|a| + |b|) exactly (rounding to nearest is
// symmetric), so one DPP-fed add per element gives the block's largest |z|.
// Both lanes compute the same sums; the maximum absorbs the duplicate.
// max |0.25 z| = RN(0.25 max |z|) because rounding is monotone, so the scaling
// is applied once at the end.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nontemporal(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <bool ROTATE>
__global__ __launch_bounds__(kThreads) void rotamax_bf16_kernel(const uint16_t* __restrict__ x,
                                                                int64_t nb,
                                                                uint32_t* __restrict__ amax_bits,
                                                                int partials, int64_t nt_end) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
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
  workgroup_max_to(m, amax_bits, partials);
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

// Pass 1 for fp32: one block per lane per iteration.
template <bool ROTATE>
__global__ __launch_bounds__(kThreads) void rotamax_f32_kernel(const float* __restrict__ x,
                                                               int64_t nb,
                                                               uint32_t* __restrict__ amax_bits,
                                                               int partials) {
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
  workgroup_max_to(m, amax_bits, partials);
}

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
  __device__ __forceinline__ int64_t operator()(int64_t b) const { return b; }
  __host__ __device__ int64_t chunks(int64_t nb) const { return (nb + kThreads - 1) / kThreads; }
  __device__ __forceinline__ int64_t first_q_byte(int64_t chunk) const { return chunk * kThreads * 8; }
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
  __device__ __forceinline__ int64_t first_q_byte(int64_t chunk) const {
    const int64_t rt = chunk / cs;
    return (rt * 128 * cb + (chunk - rt * cs) * 16) * 8;
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
  __device__ __forceinline__ bool locate(int64_t chunk, int sub, uint32_t tid, int64_t, int64_t* b,
                                         int64_t* si) const {
    const int64_t rt = chunk / cs;
    const uint32_t r = static_cast<uint32_t>(rt * 128 + sub * 16 + (tid >> 4));
    const uint32_t c = static_cast<uint32_t>(chunk - rt * cs) * 16 + (tid & 15u);
    if (r >= rows || c >= cb) return false;
    *b = static_cast<int64_t>(r) * cb + c;
    *si = place(r & 127u, c & 15u, 4);  // byte within the chunk's tiles
    return true;
  }
  // The chunk's tiles (rt, 4 c16 .. 4 c16 + 3) are consecutive in memory.
  __device__ __forceinline__ void chunk_tiles(int64_t chunk, int64_t* first_byte, int* ntiles) const {
    const int64_t rt = chunk / cs, ct0 = (chunk - rt * cs) * 4;
    *first_byte = (rt * ctiles + ct0) * 512;
    *ntiles = static_cast<int>(ctiles - ct0 < 4 ? ctiles - ct0 : 4);
  }
};

// When pass 1 leaves its per-workgroup maxima at the head of q_out, every
// pass-2 workgroup reads them in its prologue and then counts itself in; a
// workgroup waits for all of them to have done so before it writes a chunk
// whose codes reach into that head.  Chunks run last-first, so the wait comes
// at the end of the few workgroups concerned, and since the others never wait
// the count always completes.  The wait is bounded: past spin_limit sleeps the
// workgroup goes on and marks the call failed with a NaN global scale.
struct HeadGuard {
  uint32_t* counters;  // null: no partials in q_out
  int64_t bytes;       // head bytes holding partials and counters
  uint32_t need;       // pass-2 workgroups
  uint32_t spin_limit;
  float* gscale_out;
};

__device__ __forceinline__ void wait_for_head(const HeadGuard& h) {
  __shared__ int timed_out;
  if (threadIdx.x < 64) {  // wave 0: one counter per lane
    uint32_t spins = 0;
    int late = 0;
    // Relaxed: acquire/release at agent scope would write back or invalidate
    // the L2 of every XCD involved on each poll.  Nothing written by other
    // workgroups is read after the wait; the waiter's stores follow the loop.
    for (;;) {
      uint32_t c = __hip_atomic_load(h.counters + threadIdx.x * kCounterStride, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
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

// Pass 2 body: each lane rotates, scales and encodes one block per iteration.
// Workgroup w handles the 256-block chunks w, w + G, w + 2G, ... (G = grid
// size), last chunk first: the chunks pass 1 read last are the likeliest to
// still be in the last-level cache.  Every step is the definition of section 2
// (hadamard_nvfp4_kernel) in binary32:
//   z     = S16 x                         (butterfly, no scaling yet)
//   a_b   = max |y| = 0.25 max |z|        (exact for any rounding, see pass 1)
//   v     = (a_b / 6) / g,  s = E4M3(min(v, 448))
//   d     = float(s) * g, or 1 when that is 0
//   code  = E2M1(y / d),  y = 0.25 z
// FAST (bf16 in the guarded range): y / d = z / (4d) exactly (the scalings by
// 4 are exact there), the divisions are corrected reciprocal products and the
// per-scale (4d, 1/(4d)) pairs come from a 128-entry table in LDS.
// Otherwise every division is a true binary32 division.
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
  if (mine > 0 && smap.locate((mine - 1) * gridDim.x + blockIdx.x, 0, threadIdx.x, nb, &b, &si))
    f->load(x, b);
}

template <typename T, bool ROTATE, bool FAST, typename SMAP>
__device__ __forceinline__ void quant_blocks(const T* __restrict__ x, int64_t nb, float g,
                                             const float2* __restrict__ tab,
                                             uint8_t* __restrict__ q, uint8_t* __restrict__ s,
                                             SMAP smap, const HeadGuard& head,
                                             const FirstBlock<T>& first) {
  const int64_t nchunks = smap.chunks(nb);
  const int64_t mine = (nchunks - blockIdx.x + gridDim.x - 1) / gridDim.x;
  const float rg = FAST ? 1.0f / g : 0.0f;
  __shared__ uint32_t stage[SMAP::kStaged ? 512 : 1];  // 4 scale tiles
  for (int64_t it = mine - 1; it >= 0; --it) {
   const int64_t chunk = it * gridDim.x + blockIdx.x;
   if (head.counters && smap.first_q_byte(chunk) < head.bytes) wait_for_head(head);
   if constexpr (SMAP::kStaged) {
     for (uint32_t i = threadIdx.x; i < 512; i += kThreads) stage[i] = 0u;
     __syncthreads();
   }
#pragma unroll 1
   for (int sub = 0; sub < SMAP::kSub; ++sub) {
    int64_t b, si;
    if (!smap.locate(chunk, sub, threadIdx.x, nb, &b, &si)) continue;
    float lo[8], hi[8];
    if (!SMAP::kStaged && it == mine - 1 && sub == 0) {  // loaded before the prologue
      first.unpack(lo, hi);
    } else {
      load_block(x, b, lo, hi);
    }
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
    *reinterpret_cast<uint2*>(q + b * 8) = make_uint2(e2m1_pack8(lo), e2m1_pack8(hi));
    if constexpr (SMAP::kStaged)
      reinterpret_cast<uint8_t*>(stage)[si] = static_cast<uint8_t>(sb);
    else
      s[si] = static_cast<uint8_t>(sb);
   }
   if constexpr (SMAP::kStaged) {
     // whole tiles, padding zeros included, in one coalesced store
     __syncthreads();
     int64_t first;
     int ntiles;
     smap.chunk_tiles(chunk, &first, &ntiles);
     uint32_t* dst = reinterpret_cast<uint32_t*>(s + first);
     for (uint32_t i = threadIdx.x; i < static_cast<uint32_t>(ntiles) * 128u; i += kThreads)
       dst[i] = stage[i];
     __syncthreads();
   }
  }
}

// amax_src: the amax word (npartials == 0) or pass 1's per-workgroup maxima
// at the head of q (npartials of them, then the counter; amax_out receives
// their maximum).
// Eight workgroups per CU (the grid size assumes it): at most 64 VGPRs.
template <typename T, bool ROTATE, typename SMAP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void rotquant_kernel(const T* __restrict__ x, int64_t nb,
                                                            const uint32_t* amax_src,
                                                            int npartials, float* __restrict__ amax_out,
                                                            uint32_t spin_limit, int allow_fast,
                                                            uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ s,
                                                            float* __restrict__ gscale_out,
                                                            SMAP smap) {
  __shared__ float2 tab[128];
  __shared__ uint32_t red[kThreads / 64];
  FirstBlock<T> first;
  if constexpr (!SMAP::kStaged) load_first(x, nb, smap, &first);  // staged: no registers to spare
  HeadGuard head{nullptr, 0, 0, spin_limit, gscale_out};
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
    uint32_t* counters = const_cast<uint32_t*>(amax_src) + counter_base(npartials);
    // every thread's read of the partials is complete (their values met at
    // the barrier) before the workgroup counts itself in; a relaxed increment
    // needs no cache write-back
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(counters + (blockIdx.x % kCounters) * kCounterStride, 1u,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (blockIdx.x == 0 && threadIdx.x == 0) *amax_out = __uint_as_float(abits);
    head = HeadGuard{counters, head_bytes(npartials), gridDim.x, spin_limit, gscale_out};
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
      quant_blocks<T, ROTATE, true>(x, nb, g, tab, q, s, smap, head, first);
      return;
    }
  }
  quant_blocks<T, ROTATE, false>(x, nb, g, tab, q, s, smap, head, first);
}

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

// ---------------------------------------------------------------- MXFP4 variant

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

// ---------------------------------------------------------------- host helpers

// Timing hook of the *_timed entry points: while one runs on this thread, its
// k-th launch (k = 0, 1, ...) goes through hipExtLaunchKernel, which records
// events[2k] when the kernel starts and events[2k + 1] when it ends.
thread_local hipEvent_t* t_events = nullptr;
thread_local int t_pairs = 0;
thread_local int t_launched = 0;

// hipLaunchKernel with the kernel's own parameter types; returns the launch status.
template <typename... KArgs, typename... Args, size_t... I>
hipError_t launch_impl(void (*k)(KArgs...), dim3 grid, dim3 block, hipStream_t st,
                       std::index_sequence<I...>, Args... args) {
  std::tuple<KArgs...> t(static_cast<KArgs>(args)...);
  void* argv[] = {static_cast<void*>(&std::get<I>(t))..., nullptr};
  if (t_events) {
    const int n = t_launched++;
    if (n < t_pairs)
      return hipExtLaunchKernel(reinterpret_cast<const void*>(k), grid, block, argv, 0, st,
                                t_events[2 * n], t_events[2 * n + 1], 0);
  }
  return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, argv, 0, st);
}

template <typename... KArgs, typename... Args>
hipError_t launch(void (*k)(KArgs...), dim3 grid, dim3 block, hipStream_t st, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
  return launch_impl(k, grid, block, st, std::index_sequence_for<KArgs...>{}, args...);
}

// Compute units of the current device, cached per device.
int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int c = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (c == 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
      c = 256;
    __atomic_store_n(&cache[dev], c, __ATOMIC_RELAXED);
  }
  return c;
}

// Positive integer from the environment, or 0.  Used to override launch
// shapes in tests (results never depend on them).
int64_t env_int(const char* name) {
  const char* v = getenv(name);
  if (!v || !*v) return 0;
  char* end = nullptr;
  const long long n = strtoll(v, &end, 10);
  return (end && *end == '\0' && n > 0) ? n : 0;
}

int clamp_grid(int64_t want, int64_t needed) {
  int64_t g = want < needed ? want : needed;
  if (g < 1) g = 1;
  if (g > (1 << 30)) g = 1 << 30;
  return static_cast<int>(g);
}

// Pass 1: 2 workgroups per compute unit, each wave streaming 8 KiB (bf16) per
// iteration; fp32: one block per lane per iteration.  Pass 1 alone runs
// about as fast with 4 or 8 per CU, but every quantize workgroup of the fused
// call reduces one maximum per pass-1 workgroup before it starts (measured
// step at 16384 x 8192: 102.8 us with 2 per CU, 103.7 with 4, 103.2 with 8).
int amax_grid(int64_t nb, bool bf16) {
  int64_t want = env_int("NVFP4RQ_AMAX_WGS");
  if (!want) want = 2LL * device_cus();
  const int64_t per_wg = bf16 ? (kThreads / 64) * 64LL * kAmaxPieces / 2 : kThreads;  // blocks
  return clamp_grid(want, (nb + per_wg - 1) / per_wg);
}

// Pass 2: 8 workgroups per compute unit, one 256-block chunk per iteration.
int quant_grid(int64_t nb) {
  int64_t want = env_int("NVFP4RQ_QUANT_WGS");
  if (!want) want = 8LL * device_cus();
  return clamp_grid(want, (nb + kThreads - 1) / kThreads);
}

int generic_grid(int64_t nb) { return clamp_grid(8LL * device_cus(), (nb + kThreads - 1) / kThreads); }

// Quarter-block kernels: 8 workgroups per compute unit, kThreads * kQuarters
// quarters per workgroup iteration.
int quarter_grid(int64_t nq) {
  const int64_t per_wg = static_cast<int64_t>(kThreads) * kQuarters;
  return clamp_grid(8LL * device_cus(), (nq + per_wg - 1) / per_wg);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

// Shape checks shared by every entry point; *nb receives the block count.
nvfp4_status check_shape(int64_t rows, int64_t cols, int64_t* nb) {
  if (rows < 0 || cols < 0 || cols % 16 != 0) return NVFP4_ERR_SHAPE;
  // largest buffer is rows * cols * 4 bytes (fp32 input or output)
  if (cols != 0 && rows > (INT64_MAX / 8) / cols) return NVFP4_ERR_SHAPE;
  *nb = rows * (cols / 16);
  return NVFP4_OK;
}

template <typename T>
nvfp4_status validate_quant(const T* x, int64_t rows, int64_t cols, int rotate, const uint8_t* q,
                            const uint8_t* s, const float* g, const float* amax, int64_t* nb,
                            bool amax_is_input, int64_t s_bytes = -1) {
  nvfp4_status st = check_shape(rows, cols, nb);
  if (st != NVFP4_OK) return st;
  const int64_t n = rows * cols;
  if ((n != 0 && (!x || !q || !s)) || !g || !amax) return NVFP4_ERR_NULL;
  if (rotate != 0 && rotate != 1) return NVFP4_ERR_ARG;
  if (n != 0 && (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4))) return NVFP4_ERR_ALIGN;
  if (!aligned(g, 4) || !aligned(amax, 4)) return NVFP4_ERR_ALIGN;
  const Range rx = range_of(x, n * static_cast<int64_t>(sizeof(T)));
  const Range rq = range_of(q, n / 2), rs = range_of(s, s_bytes < 0 ? n / 16 : s_bytes);
  const Range rg = range_of(g, 4), ra = range_of(amax, 4);
  const Range outs[4] = {rq, rs, rg, ra};
  const int n_out = amax_is_input ? 3 : 4;
  for (int i = 0; i < 4; ++i) {
    if (overlap(outs[i], rx)) return NVFP4_ERR_ARG;
    for (int j = i + 1; j < 4; ++j)
      if ((i < n_out || j < n_out) && overlap(outs[i], outs[j])) return NVFP4_ERR_ARG;
  }
  return NVFP4_OK;
}

// partials == 1: pass 1 stores its per-workgroup maxima (and a cleared
// counter) at bits[0 .. grid] instead of an atomicMax into bits[0].
int amax_grid_for(const uint16_t*, int64_t nb) { return amax_grid(nb, true); }
int amax_grid_for(const float*, int64_t nb) { return amax_grid(nb, false); }

hipError_t launch_rotamax(const uint16_t* x, int64_t nb, int rotate, uint32_t* bits, int partials,
                          hipStream_t st) {
  const dim3 grid(amax_grid(nb, true));
  // The quantize pass walks the tensor last-first and finds the part pass 1
  // read last in the 256 MB last-level cache; the part before the last
  // kLastLevelKeep bytes would be evicted before the quantize pass got to it,
  // so pass 1 streams it with non-temporal loads (measured at 16384 x 8192:
  // 1 us off pass 1, nothing lost in pass 2; streaming more costs pass 2 its
  // cache hits).
  const int64_t keep_mb = env_int("NVFP4RQ_LLC_KEEP_MB");
  const int64_t keep_pieces = (keep_mb ? keep_mb << 20 : kLastLevelKeep) / 16;
  const int64_t nt_end = 2 * nb > keep_pieces ? 2 * nb - keep_pieces : 0;
  return rotate ? launch(rotamax_bf16_kernel<true>, grid, dim3(kThreads), st, x, nb, bits, partials, nt_end)
                : launch(rotamax_bf16_kernel<false>, grid, dim3(kThreads), st, x, nb, bits, partials,
                         nt_end);
}

hipError_t launch_rotamax(const float* x, int64_t nb, int rotate, uint32_t* bits, int partials,
                          hipStream_t st) {
  const dim3 grid(amax_grid(nb, false));
  return rotate ? launch(rotamax_f32_kernel<true>, grid, dim3(kThreads), st, x, nb, bits, partials)
                : launch(rotamax_f32_kernel<false>, grid, dim3(kThreads), st, x, nb, bits, partials);
}

template <typename T>
nvfp4_status enqueue_rotamax(const T* x, int64_t nb, int rotate, float* amax, hipStream_t st) {
  uint32_t* bits = reinterpret_cast<uint32_t*>(amax);
  if (launch(zero_word_kernel, dim3(1), dim3(1), st, bits) != hipSuccess) return NVFP4_ERR_HIP;
  if (nb == 0) return NVFP4_OK;
  return launch_rotamax(x, nb, rotate, bits, 0, st) == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

// Pass 2.  npartials == 0: the amax is the word at amax_src.  Otherwise
// amax_src holds npartials per-workgroup maxima and the counter (at the head
// of q) and the kernel writes their maximum to amax_out.
template <typename T, typename SMAP = RowMajorScales>
nvfp4_status enqueue_quant(const T* x, int64_t nb, int rotate, const uint32_t* amax_src,
                           int npartials, float* amax_out, uint8_t* q, uint8_t* s, float* g,
                           hipStream_t st, SMAP smap = SMAP{}) {
  const int allow_fast = env_int("NVFP4RQ_EXACT_ONLY") ? 0 : 1;
  const int64_t spin_env = env_int("NVFP4RQ_SPIN_LIMIT");
  const uint32_t spin_limit = spin_env > 0 ? static_cast<uint32_t>(spin_env) : (1u << 26);
  const dim3 grid(quant_grid(smap.chunks(nb) * kThreads));
  const hipError_t e =
      rotate ? launch(rotquant_kernel<T, true, SMAP>, grid, dim3(kThreads), st, x, nb, amax_src,
                      npartials, amax_out, spin_limit, allow_fast, q, s, g, smap)
             : launch(rotquant_kernel<T, false, SMAP>, grid, dim3(kThreads), st, x, nb, amax_src,
                      npartials, amax_out, spin_limit, allow_fast, q, s, g, smap);
  return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

// Both passes.  When q_out has room (8 nb bytes against head_bytes: from
// about 1040 blocks up), pass 1 leaves per-workgroup maxima and cleared counters at
// the head of q_out (which pass 2 overwrites last), so no word has to be
// zeroed first; smaller tensors take the zeroed-word path.
template <typename T, typename SMAP = RowMajorScales>
nvfp4_status enqueue_both(const T* x, int64_t nb, int rotate, uint8_t* q, uint8_t* s, float* g,
                          float* amax, hipStream_t st, SMAP smap = SMAP{}) {
  const int g1 = amax_grid_for(x, nb);
  if (nb == 0 || head_bytes(g1) > 8 * nb || env_int("NVFP4RQ_ZEROED_AMAX")) {
    nvfp4_status r = enqueue_rotamax(x, nb, rotate, amax, st);
    if (r != NVFP4_OK) return r;
    return enqueue_quant(x, nb, rotate, reinterpret_cast<const uint32_t*>(amax), 0, amax, q, s, g, st,
                         smap);
  }
  uint32_t* head = reinterpret_cast<uint32_t*>(q);
  if (launch_rotamax(x, nb, rotate, head, 1, st) != hipSuccess) return NVFP4_ERR_HIP;
  return enqueue_quant(x, nb, rotate, head, g1, amax, q, s, g, st, smap);
}

// Size of the swizzled scale buffer for a [rows, cols] tensor; -1 for a bad
// shape or more than 2^32 - 1 blocks.
int64_t swizzled_bytes(int64_t rows, int64_t cols) {
  int64_t nb = 0;
  if (check_shape(rows, cols, &nb) != NVFP4_OK || nb > 0xFFFFFFFFLL) return -1;
  const int64_t cb = cols / 16;
  return ((rows + 127) / 128) * ((cb + 3) / 4) * 512;
}

template <typename T>
nvfp4_status rotquant_swizzled(const T* x, int64_t rows, int64_t cols, int rotate, uint8_t* q,
                               uint8_t* s, float* g, float* amax, hipStream_t st) {
  const int64_t sbytes = swizzled_bytes(rows, cols);
  if (sbytes < 0) return NVFP4_ERR_SHAPE;
  int64_t nb = 0;
  nvfp4_status r = validate_quant(x, rows, cols, rotate, q, s, g, amax, &nb, false, sbytes);
  if (r != NVFP4_OK) return r;
  const uint32_t cb = static_cast<uint32_t>(cols / 16), ctiles = (cb + 3) / 4;
  return enqueue_both(x, nb, rotate, q, s, g, amax, st, SwizzledScales{rows, cb, ctiles, (cb + 15) / 16});
}

template <typename T>
nvfp4_status rotquant(const T* x, int64_t rows, int64_t cols, int rotate, uint8_t* q, uint8_t* s,
                      float* g, float* amax, hipStream_t st) {
  int64_t nb = 0;
  nvfp4_status r = validate_quant(x, rows, cols, rotate, q, s, g, amax, &nb, false);
  if (r != NVFP4_OK) return r;
  return enqueue_both(x, nb, rotate, q, s, g, amax, st);
}

template <typename T>
nvfp4_status rotamax(const T* x, int64_t rows, int64_t cols, int rotate, float* amax,
                     hipStream_t st) {
  int64_t nb = 0;
  nvfp4_status r = check_shape(rows, cols, &nb);
  if (r != NVFP4_OK) return r;
  const int64_t n = rows * cols;
  if ((n != 0 && !x) || !amax) return NVFP4_ERR_NULL;
  if (rotate != 0 && rotate != 1) return NVFP4_ERR_ARG;
  if ((n != 0 && !aligned(x, 16)) || !aligned(amax, 4)) return NVFP4_ERR_ALIGN;
  if (overlap(range_of(amax, 4), range_of(x, n * static_cast<int64_t>(sizeof(T)))))
    return NVFP4_ERR_ARG;
  return enqueue_rotamax(x, nb, rotate, amax, st);
}

template <typename T>
nvfp4_status quant_from_amax(const T* x, int64_t rows, int64_t cols, int rotate,
                             const float* amax, uint8_t* q, uint8_t* s, float* g,
                             hipStream_t st) {
  int64_t nb = 0;
  nvfp4_status r = validate_quant(x, rows, cols, rotate, q, s, g, amax, &nb, true);
  if (r != NVFP4_OK) return r;
  return enqueue_quant(x, nb, rotate, reinterpret_cast<const uint32_t*>(amax), 0, nullptr, q, s, g,
                       st);
}


template <typename T>
nvfp4_status mx_rotquant(const T* x, int64_t rows, int64_t cols, int rotate, uint8_t* q, uint8_t* s,
                         hipStream_t st) {
  if (rows < 0 || cols < 0 || cols % 32 != 0) return NVFP4_ERR_SHAPE;
  int64_t nb = 0;
  nvfp4_status r = check_shape(rows, cols, &nb);
  if (r != NVFP4_OK) return r;
  const int64_t n = rows * cols;
  if (n != 0 && (!x || !q || !s)) return NVFP4_ERR_NULL;
  if (rotate != 0 && rotate != 1) return NVFP4_ERR_ARG;
  if (n != 0 && (!aligned(x, 16) || !aligned(q, 16))) return NVFP4_ERR_ALIGN;
  const Range rx = range_of(x, n * static_cast<int64_t>(sizeof(T)));
  const Range rq = range_of(q, n / 2), rs = range_of(s, n / 32);
  if (overlap(rq, rx) || overlap(rs, rx) || overlap(rq, rs)) return NVFP4_ERR_ARG;
  const int64_t nb32 = n / 32;
  if (nb32 == 0) return NVFP4_OK;
  const dim3 grid(quant_grid(nb32));
  const hipError_t e = rotate ? launch(mx_quant_kernel<T, true>, grid, dim3(kThreads), st, x, nb32, q, s)
                              : launch(mx_quant_kernel<T, false>, grid, dim3(kThreads), st, x, nb32, q, s);
  return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}


template <typename T>
nvfp4_status rotate_only(const T* x, int64_t rows, int64_t cols, float* y, hipStream_t st) {
  int64_t nb = 0;
  nvfp4_status r = check_shape(rows, cols, &nb);
  if (r != NVFP4_OK) return r;
  const int64_t n = rows * cols;
  if (n != 0 && (!x || !y)) return NVFP4_ERR_NULL;
  if (n != 0 && (!aligned(x, 16) || !aligned(y, 16))) return NVFP4_ERR_ALIGN;
  if (overlap(range_of(x, n * static_cast<int64_t>(sizeof(T))), range_of(y, n * 4)))
    return NVFP4_ERR_ARG;
  if (nb == 0) return NVFP4_OK;
  const int64_t nq = 4 * nb;
  return launch(rotate_kernel<T>, dim3(quarter_grid(nq)), dim3(kThreads), st, x, nq, y) == hipSuccess
             ? NVFP4_OK
             : NVFP4_ERR_HIP;
}
template <typename SMAP>
nvfp4_status dequant(const uint8_t* q, const uint8_t* s, const float* gscale, int64_t rows,
                     int64_t cols, int rotate, float* y_out, hipStream_t stream, int64_t s_bytes,
                     SMAP smap) {
  int64_t nb = 0;
  nvfp4_status r = check_shape(rows, cols, &nb);
  if (r != NVFP4_OK) return r;
  const int64_t n = rows * cols;
  if ((n != 0 && (!q || !s || !y_out)) || !gscale) return NVFP4_ERR_NULL;
  if (rotate != 0 && rotate != 1) return NVFP4_ERR_ARG;
  if ((n != 0 && (!aligned(q, 8) || !aligned(y_out, 16))) || !aligned(gscale, 4))
    return NVFP4_ERR_ALIGN;
  const Range ry = range_of(y_out, n * 4);
  if (overlap(ry, range_of(q, n / 2)) || overlap(ry, range_of(s, s_bytes < 0 ? n / 16 : s_bytes)) ||
      overlap(ry, range_of(gscale, 4)))
    return NVFP4_ERR_ARG;
  if (nb == 0) return NVFP4_OK;
  const int64_t nq = 4 * nb;
  if (launch(dequant_kernel<SMAP>, dim3(quarter_grid(nq)), dim3(kThreads), stream, q, s, gscale, nq,
             rotate, y_out, smap) != hipSuccess)
    return NVFP4_ERR_HIP;
  return NVFP4_OK;
}

}  // namespace

// ---------------------------------------------------------------- C ABI

extern "C" {

nvfp4_status nvfp4_rotquant(const uint16_t* x_bf16, int64_t rows, int64_t cols, int rotate,
                            uint8_t* q_out, uint8_t* s_out, float* gscale_out, float* amax_out,
                            hipStream_t stream) {
  return rotquant(x_bf16, rows, cols, rotate, q_out, s_out, gscale_out, amax_out, stream);
}

nvfp4_status nvfp4_rotquant_timed(const uint16_t* x_bf16, int64_t rows, int64_t cols, int rotate,
                                  uint8_t* q_out, uint8_t* s_out, float* gscale_out,
                                  float* amax_out, hipStream_t stream, hipEvent_t* events,
                                  int npairs, int* nkernels) {
  if (!events || npairs < 1 || !nkernels) return NVFP4_ERR_NULL;
  t_events = events;
  t_pairs = npairs;
  t_launched = 0;
  const nvfp4_status r =
      rotquant(x_bf16, rows, cols, rotate, q_out, s_out, gscale_out, amax_out, stream);
  *nkernels = t_launched;
  t_events = nullptr;
  t_pairs = 0;
  t_launched = 0;
  return r;
}

nvfp4_status nvfp4_rotquant_f32(const float* x, int64_t rows, int64_t cols, int rotate,
                                uint8_t* q_out, uint8_t* s_out, float* gscale_out,
                                float* amax_out, hipStream_t stream) {
  return rotquant(x, rows, cols, rotate, q_out, s_out, gscale_out, amax_out, stream);
}

nvfp4_status nvfp4_rotamax(const uint16_t* x_bf16, int64_t rows, int64_t cols, int rotate,
                           float* amax_out, hipStream_t stream) {
  return rotamax(x_bf16, rows, cols, rotate, amax_out, stream);
}

nvfp4_status nvfp4_rotamax_f32(const float* x, int64_t rows, int64_t cols, int rotate,
                               float* amax_out, hipStream_t stream) {
  return rotamax(x, rows, cols, rotate, amax_out, stream);
}

nvfp4_status nvfp4_quant_from_amax(const uint16_t* x_bf16, int64_t rows, int64_t cols,
                                   int rotate, const float* amax_in, uint8_t* q_out,
                                   uint8_t* s_out, float* gscale_out, hipStream_t stream) {
  return quant_from_amax(x_bf16, rows, cols, rotate, amax_in, q_out, s_out, gscale_out, stream);
}

nvfp4_status nvfp4_quant_from_amax_f32(const float* x, int64_t rows, int64_t cols, int rotate,
                                       const float* amax_in, uint8_t* q_out, uint8_t* s_out,
                                       float* gscale_out, hipStream_t stream) {
  return quant_from_amax(x, rows, cols, rotate, amax_in, q_out, s_out, gscale_out, stream);
}

nvfp4_status nvfp4_dequant(const uint8_t* q, const uint8_t* s, const float* gscale, int64_t rows,
                           int64_t cols, int rotate, float* y_out, hipStream_t stream) {
  return dequant(q, s, gscale, rows, cols, rotate, y_out, stream, -1, RowMajorScales{});
}

int64_t nvfp4_swizzled_scale_bytes(int64_t rows, int64_t cols) { return swizzled_bytes(rows, cols); }

nvfp4_status nvfp4_rotquant_swizzled(const uint16_t* x_bf16, int64_t rows, int64_t cols, int rotate,
                                     uint8_t* q_out, uint8_t* s_out, float* gscale_out,
                                     float* amax_out, hipStream_t stream) {
  return rotquant_swizzled(x_bf16, rows, cols, rotate, q_out, s_out, gscale_out, amax_out, stream);
}

nvfp4_status nvfp4_rotquant_swizzled_f32(const float* x, int64_t rows, int64_t cols, int rotate,
                                         uint8_t* q_out, uint8_t* s_out, float* gscale_out,
                                         float* amax_out, hipStream_t stream) {
  return rotquant_swizzled(x, rows, cols, rotate, q_out, s_out, gscale_out, amax_out, stream);
}

nvfp4_status nvfp4_dequant_swizzled(const uint8_t* q, const uint8_t* s, const float* gscale,
                                    int64_t rows, int64_t cols, int rotate, float* y_out,
                                    hipStream_t stream) {
  const int64_t sbytes = swizzled_bytes(rows, cols);
  if (sbytes < 0) return NVFP4_ERR_SHAPE;
  const uint32_t cb = static_cast<uint32_t>(cols / 16);
  return dequant(q, s, gscale, rows, cols, rotate, y_out, stream, sbytes,
                 SwizzledScales{rows, cb, (cb + 3) / 4, (cb + 15) / 16});
}

nvfp4_status nvfp4_rotate16(const uint16_t* x_bf16, int64_t rows, int64_t cols, float* y_out,
                            hipStream_t stream) {
  return rotate_only(x_bf16, rows, cols, y_out, stream);
}

nvfp4_status nvfp4_rotate16_f32(const float* x, int64_t rows, int64_t cols, float* y_out,
                                hipStream_t stream) {
  return rotate_only(x, rows, cols, y_out, stream);
}

nvfp4_status mxfp4_rotquant(const uint16_t* x_bf16, int64_t rows, int64_t cols, int rotate,
                            uint8_t* q_out, uint8_t* s_out, hipStream_t stream) {
  return mx_rotquant(x_bf16, rows, cols, rotate, q_out, s_out, stream);
}

nvfp4_status mxfp4_rotquant_f32(const float* x, int64_t rows, int64_t cols, int rotate,
                                uint8_t* q_out, uint8_t* s_out, hipStream_t stream) {
  return mx_rotquant(x, rows, cols, rotate, q_out, s_out, stream);
}

nvfp4_status mxfp4_dequant(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols,
                           int rotate, float* y_out, hipStream_t stream) {
  if (rows < 0 || cols < 0 || cols % 32 != 0) return NVFP4_ERR_SHAPE;
  int64_t nb = 0;
  nvfp4_status r = check_shape(rows, cols, &nb);
  if (r != NVFP4_OK) return r;
  const int64_t n = rows * cols;
  if (n != 0 && (!q || !s || !y_out)) return NVFP4_ERR_NULL;
  if (rotate != 0 && rotate != 1) return NVFP4_ERR_ARG;
  if (n != 0 && (!aligned(q, 16) || !aligned(y_out, 16))) return NVFP4_ERR_ALIGN;
  const Range ry = range_of(y_out, n * 4);
  if (overlap(ry, range_of(q, n / 2)) || overlap(ry, range_of(s, n / 32))) return NVFP4_ERR_ARG;
  const int64_t nb32 = n / 32;
  if (nb32 == 0) return NVFP4_OK;
  const int64_t nq = 8 * nb32;
  if (launch(mx_dequant_kernel, dim3(quarter_grid(nq)), dim3(kThreads), stream, q, s, nq, rotate,
             y_out) != hipSuccess)
    return NVFP4_ERR_HIP;
  return NVFP4_OK;
}

const char* nvfp4_status_string(nvfp4_status status) {
  switch (status) {
    case NVFP4_OK: return "success";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "bad shape: rows and cols must be >= 0, cols a multiple of 16, size in range";
    case NVFP4_ERR_ALIGN: return "a pointer is not aligned as its argument requires";
    case NVFP4_ERR_ARG: return "bad argument: rotate must be 0 or 1 and buffers must not overlap";
    case NVFP4_ERR_HIP: return "the HIP runtime rejected a kernel launch";
  }
  return "unknown status";
}

}  // extern "C"
