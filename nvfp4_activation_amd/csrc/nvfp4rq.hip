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
#include <cstdint>
#include <tuple>
#include <utility>

#include "nvfp4rq.h"

namespace {

constexpr int kThreads = 256;        // 4 waves of 64
constexpr int kMaxGrid = 8192;       // grid-stride beyond this

// ---------------------------------------------------------------- loads

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// One 16-value block as binary32 (bf16 widening is a shift: exact).
__device__ __forceinline__ void load_block(const uint16_t* __restrict__ x, int64_t b, float v[16]) {
  const uint4* p = reinterpret_cast<const uint4*>(x + b * 16);
  uint4 a = p[0];
  uint4 c = p[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
}

__device__ __forceinline__ void load_block(const float* __restrict__ x, int64_t b, float v[16]) {
  const float4* p = reinterpret_cast<const float4*>(x + b * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float4 t = p[i];
    v[4 * i] = t.x;
    v[4 * i + 1] = t.y;
    v[4 * i + 2] = t.z;
    v[4 * i + 3] = t.w;
  }
}

// ---------------------------------------------------------------- rotation

// z <- S16 z with S16 the unnormalised Sylvester matrix: butterfly stages with
// strides 1, 2, 4, 8, each pair (a, b) -> (a + b, a - b).  H16 = S16 / 4
// (section 1 and section 2, hadamard16).
__device__ __forceinline__ void butterfly16(float z[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const float a = z[i];
        const float b = z[i + h];
        z[i] = a + b;
        z[i + h] = a - b;
      }
    }
  }
}

// ---------------------------------------------------------------- scalar encodings

// min(round-to-nearest-even onto E4M3, 448) for v >= 0, as the E4M3FN byte.
// Normal range: round the binary32 mantissa to 3 bits (add half an E4M3 ulp
// minus one, plus the lowest kept bit, then truncate); the carry moves into
// the exponent by itself.  Below 2^-6 the quantum is 2^-9.
__device__ __forceinline__ uint32_t e4m3_byte(float v) {
  if (!(v < 448.0f)) return 0x7Eu;
  if (v < 0x1p-6f) return static_cast<uint32_t>(__builtin_rintf(v * 512.0f));
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  return (u >> 20) - (120u << 3);   // rebias 127 -> 7 on the exponent field
}

__device__ __forceinline__ float e4m3_value(uint32_t b) {
  if (b < 8u) return static_cast<float>(b) * 0x1p-9f;
  return __uint_as_float((b + (120u << 3)) << 20);
}

// E2M1 code: midpoint compares, strict and non-strict alternating so that an
// exact midpoint takes the even code; bit 3 when v < 0 (section 2, _e2m1_code).
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = __builtin_fabsf(v);
  uint32_t m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) +
               (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return m + (v < 0.0f ? 8u : 0u);
}

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t u) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(u), off, 64));
    u = u > o ? u : o;
  }
  return u;
}

// ---------------------------------------------------------------- kernels

__global__ void zero_word_kernel(uint32_t* __restrict__ w) { *w = 0u; }

// Pass 1: rotated global amax (section 2: the global scale needs the amax of
// the whole rotated tensor before any block is scaled).
template <typename T>
__global__ __launch_bounds__(kThreads) void rotamax_kernel(const T* __restrict__ x, int64_t nb,
                                                           int rotate,
                                                           uint32_t* __restrict__ amax_bits) {
  uint32_t m = 0u;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; b < nb;
       b += stride) {
    float v[16];
    load_block(x, b, v);
    if (rotate) butterfly16(v);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t a = __float_as_uint(v[i]) & 0x7FFFFFFFu;
      m = m > a ? m : a;
    }
  }
  // max |0.25 z| = 0.25 max |z| exactly: rounding to nearest is monotone and
  // the scaling by 0.25 commutes with it.
  if (rotate) m = __float_as_uint(0.25f * __uint_as_float(m));
  m = wave_max_u32(m);
  __shared__ uint32_t part[kThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) part[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = part[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) r = r > part[i] ? r : part[i];
    atomicMax(amax_bits, r);
  }
}

// Global scale from the amax: (A / 6) / 448 in binary32, 1.0 when zero
// (section 1 table; section 2, quantize).
__device__ __forceinline__ float global_scale(float amax) {
  float g = (amax / 6.0f) / 448.0f;
  return g == 0.0f ? 1.0f : g;
}

// Pass 2: rotate + quantize, one block per lane per iteration (section 2,
// hadamard_nvfp4_kernel).
template <typename T>
__global__ __launch_bounds__(kThreads) void rotquant_kernel(const T* __restrict__ x, int64_t nb,
                                                            int rotate,
                                                            const uint32_t* __restrict__ amax_bits,
                                                            uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ s,
                                                            float* __restrict__ gscale_out) {
  const float g = global_scale(__uint_as_float(*amax_bits));
  if (blockIdx.x == 0 && threadIdx.x == 0) *gscale_out = g;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; b < nb;
       b += stride) {
    float y[16];
    load_block(x, b, y);
    if (rotate) {
      butterfly16(y);
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = 0.25f * y[i];
    }
    float ab = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ab = __builtin_fmaxf(ab, __builtin_fabsf(y[i]));
    const float v = (ab / 6.0f) / g;
    const uint32_t sb = e4m3_byte(v);
    const float sf = e4m3_value(sb) * g;
    const float d = (sf == 0.0f) ? 1.0f : sf;
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i >> 3] |= e2m1_code(y[i] / d) << (4 * (i & 7));
    *reinterpret_cast<uint2*>(q + b * 8) = make_uint2(w[0], w[1]);
    s[b] = static_cast<uint8_t>(sb);
  }
}

// Dequantize (section 2, dequantize): +-GRID[c & 7] * fl(float(s) * g), then
// the same butterfly and * 0.25 when rotated (H16 is symmetric, so H16^T is
// the forward transform).
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* __restrict__ q,
                                                           const uint8_t* __restrict__ s,
                                                           const float* __restrict__ gscale,
                                                           int64_t nb, int rotate,
                                                           float* __restrict__ y) {
  constexpr float kGrid[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  const float g = *gscale;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; b < nb;
       b += stride) {
    const uint2 w = *reinterpret_cast<const uint2*>(q + b * 8);
    const float sf = e4m3_value(s[b]) * g;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t c = ((i < 8 ? w.x : w.y) >> (4 * (i & 7))) & 15u;
      const float mag = kGrid[c & 7u];
      v[i] = ((c & 8u) ? -mag : mag) * sf;
    }
    if (rotate) {
      butterfly16(v);
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0.25f * v[i];
    }
    float4* o = reinterpret_cast<float4*>(y + b * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
}

// ---------------------------------------------------------------- host helpers

// hipLaunchKernel with the kernel's own parameter types; returns the launch status.
template <typename... KArgs, typename... Args, size_t... I>
hipError_t launch_impl(void (*k)(KArgs...), dim3 grid, dim3 block, hipStream_t st,
                       std::index_sequence<I...>, Args... args) {
  std::tuple<KArgs...> t(static_cast<KArgs>(args)...);
  void* argv[] = {static_cast<void*>(&std::get<I>(t))..., nullptr};
  return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, argv, 0, st);
}

template <typename... KArgs, typename... Args>
hipError_t launch(void (*k)(KArgs...), dim3 grid, dim3 block, hipStream_t st, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
  return launch_impl(k, grid, block, st, std::index_sequence_for<KArgs...>{}, args...);
}

int grid_for(int64_t nb) {
  int64_t g = (nb + kThreads - 1) / kThreads;
  if (g < 1) g = 1;
  if (g > kMaxGrid) g = kMaxGrid;
  return static_cast<int>(g);
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
                            bool amax_is_input) {
  nvfp4_status st = check_shape(rows, cols, nb);
  if (st != NVFP4_OK) return st;
  const int64_t n = rows * cols;
  if ((n != 0 && (!x || !q || !s)) || !g || !amax) return NVFP4_ERR_NULL;
  if (rotate != 0 && rotate != 1) return NVFP4_ERR_ARG;
  if (n != 0 && (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4))) return NVFP4_ERR_ALIGN;
  if (!aligned(g, 4) || !aligned(amax, 4)) return NVFP4_ERR_ALIGN;
  const Range rx = range_of(x, n * static_cast<int64_t>(sizeof(T)));
  const Range rq = range_of(q, n / 2), rs = range_of(s, n / 16);
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

template <typename T>
nvfp4_status enqueue_rotamax(const T* x, int64_t nb, int rotate, float* amax, hipStream_t st) {
  uint32_t* bits = reinterpret_cast<uint32_t*>(amax);
  if (launch(zero_word_kernel, dim3(1), dim3(1), st, bits) != hipSuccess) return NVFP4_ERR_HIP;
  if (nb == 0) return NVFP4_OK;
  if (launch(rotamax_kernel<T>, dim3(grid_for(nb)), dim3(kThreads), st, x, nb, rotate, bits) !=
      hipSuccess)
    return NVFP4_ERR_HIP;
  return NVFP4_OK;
}

template <typename T>
nvfp4_status enqueue_quant(const T* x, int64_t nb, int rotate, const float* amax, uint8_t* q,
                           uint8_t* s, float* g, hipStream_t st) {
  const uint32_t* bits = reinterpret_cast<const uint32_t*>(amax);
  if (launch(rotquant_kernel<T>, dim3(grid_for(nb)), dim3(kThreads), st, x, nb, rotate, bits, q,
             s, g) != hipSuccess)
    return NVFP4_ERR_HIP;
  return NVFP4_OK;
}

template <typename T>
nvfp4_status rotquant(const T* x, int64_t rows, int64_t cols, int rotate, uint8_t* q, uint8_t* s,
                      float* g, float* amax, hipStream_t st) {
  int64_t nb = 0;
  nvfp4_status r = validate_quant(x, rows, cols, rotate, q, s, g, amax, &nb, false);
  if (r != NVFP4_OK) return r;
  r = enqueue_rotamax(x, nb, rotate, amax, st);
  if (r != NVFP4_OK) return r;
  return enqueue_quant(x, nb, rotate, amax, q, s, g, st);
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
  return enqueue_quant(x, nb, rotate, amax, q, s, g, st);
}

}  // namespace

// ---------------------------------------------------------------- C ABI

extern "C" {

nvfp4_status nvfp4_rotquant(const uint16_t* x_bf16, int64_t rows, int64_t cols, int rotate,
                            uint8_t* q_out, uint8_t* s_out, float* gscale_out, float* amax_out,
                            hipStream_t stream) {
  return rotquant(x_bf16, rows, cols, rotate, q_out, s_out, gscale_out, amax_out, stream);
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
  int64_t nb = 0;
  nvfp4_status r = check_shape(rows, cols, &nb);
  if (r != NVFP4_OK) return r;
  const int64_t n = rows * cols;
  if ((n != 0 && (!q || !s || !y_out)) || !gscale) return NVFP4_ERR_NULL;
  if (rotate != 0 && rotate != 1) return NVFP4_ERR_ARG;
  if ((n != 0 && (!aligned(q, 8) || !aligned(y_out, 16))) || !aligned(gscale, 4))
    return NVFP4_ERR_ALIGN;
  const Range ry = range_of(y_out, n * 4);
  if (overlap(ry, range_of(q, n / 2)) || overlap(ry, range_of(s, n / 16)) ||
      overlap(ry, range_of(gscale, 4)))
    return NVFP4_ERR_ARG;
  if (nb == 0) return NVFP4_OK;
  if (launch(dequant_kernel, dim3(grid_for(nb)), dim3(kThreads), stream, q, s, gscale, nb, rotate,
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
