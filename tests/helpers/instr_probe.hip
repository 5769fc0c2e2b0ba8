// GPU side of the instruction checks (test code): runs the library's own
// conversion and division helpers (nvfp4rq_device.hpp) over ranges of
// binary32 bit patterns so that the tests can compare every output with a CPU
// computation.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "nvfp4rq_device.hpp"

using namespace nvfp4rq;

// one byte per input: the E2M1 code e2m1_pack8 gives to value base + i
__global__ void e2m1_kernel(uint32_t base, uint32_t n, uint8_t* __restrict__ out) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = __uint_as_float(base + i);
  float q[8] = {v, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  out[i] = static_cast<uint8_t>(e2m1_pack8(q) & 15u);
}

// one byte per input: e4m3_byte(base + i)
__global__ void e4m3_kernel(uint32_t base, uint32_t n, uint8_t* __restrict__ out) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  out[i] = static_cast<uint8_t>(e4m3_byte(__uint_as_float(base + i)));
}

// 16 values -> 8 packed bytes, to check the nibble order
__global__ void pack_kernel(const float* __restrict__ v, uint32_t* __restrict__ out) {
  float a[8], b[8];
  for (int i = 0; i < 8; ++i) { a[i] = v[i]; b[i] = v[8 + i]; }
  out[0] = e2m1_pack8(a);
  out[1] = e2m1_pack8(b);
}

// all 256 E4M3 byte values -> float (e4m3_value); every byte at each of the
// four positions of a word -> its two E2M1 values (e2m1_pair), the other
// bytes holding junk: e2m1[2 (256 pos + byte) + k]
__global__ void values_kernel(float* __restrict__ e4m3, float* __restrict__ e2m1) {
  const uint32_t i = threadIdx.x;
  e4m3[i] = e4m3_value(i);
  const uint32_t junk = 0xA5C3963Cu;
#pragma unroll
  for (int pos = 0; pos < 4; ++pos) {
    const uint32_t w = (junk & ~(0xFFu << (8 * pos))) | (i << (8 * pos));
    float2 v;
    if (pos == 0) v = e2m1_pair<0>(w);
    else if (pos == 1) v = e2m1_pair<1>(w);
    else if (pos == 2) v = e2m1_pair<2>(w);
    else v = e2m1_pair<3>(w);
    e2m1[2 * (256 * pos + i)] = v.x;
    e2m1[2 * (256 * pos + i) + 1] = v.y;
  }
}

// the fast path's global scale (two corrected products) of amax base + i * stride
__global__ void gscale_kernel(uint32_t base, uint32_t stride, uint32_t n, uint32_t* __restrict__ out) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  out[i] = __float_as_uint(global_scale_corrected(__uint_as_float(base + i * stride)));
}

// the two words of the reciprocal table entry for D = base + i * stride
__global__ void recip2_kernel(uint32_t base, uint32_t stride, uint32_t n, uint32_t* __restrict__ out) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float2 r = recip2_corrected(__uint_as_float(base + i * stride));
  out[2 * i] = __float_as_uint(r.x);
  out[2 * i + 1] = __float_as_uint(r.y);
}

extern "C" {
// out: n words; base + (n - 1) * stride must not wrap (the caller checks)
int probe_gscale(uint32_t base, uint32_t stride, uint32_t n, uint32_t* out, hipStream_t st) {
  gscale_kernel<<<(n + 255) / 256, 256, 0, st>>>(base, stride, n, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
// out: 2 n words
int probe_recip2(uint32_t base, uint32_t stride, uint32_t n, uint32_t* out, hipStream_t st) {
  recip2_kernel<<<(n + 255) / 256, 256, 0, st>>>(base, stride, n, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
int probe_e2m1(uint32_t base, uint32_t n, uint8_t* out, hipStream_t st) {
  e2m1_kernel<<<(n + 255) / 256, 256, 0, st>>>(base, n, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
int probe_e4m3(uint32_t base, uint32_t n, uint8_t* out, hipStream_t st) {
  e4m3_kernel<<<(n + 255) / 256, 256, 0, st>>>(base, n, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
int probe_pack(const float* v, uint32_t* out, hipStream_t st) {
  pack_kernel<<<1, 1, 0, st>>>(v, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
// e4m3: 256 floats; e2m1: 2048 floats
int probe_values(float* e4m3, float* e2m1, hipStream_t st) {
  values_kernel<<<1, 256, 0, st>>>(e4m3, e2m1);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
}
