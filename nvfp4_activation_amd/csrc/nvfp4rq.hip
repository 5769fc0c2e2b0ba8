// Fused block-Hadamard rotation + NVFP4 activation quantization for gfx950:
// host side and C ABI of libnvfp4rq.  The kernels are in common.hpp (shared
// constants, reductions, loads), pass1.hpp (rotated amax), pass2.hpp
// (quantize), mxfp4.hpp (MXFP4 variant) and elementwise.hpp (decode, rotation
// alone); all are compiled in this one translation unit.
//
// Method: page "A Fused Hadamard + NVFP4 Quantization Kernel in Triton"
// (kanthi.in), sections 1-3; stored layout: page "NVFP4 Quantization"
// (atlas-docs), section "The numeric format".  The C ABI and its contract are
// in include/nvfp4rq.h.
//
// The fused call is two kernels:
//   pass 1  reads every 16-value block, rotates it in registers, and keeps
//           the running max |y| as binary32 bits (non-negative floats order
//           like unsigned integers, so the max is exact and independent of
//           the reduction order); each workgroup stores its maximum at the
//           head of q_out (or, for small tensors and the pass-level entry
//           point, does one atomicMax into a zeroed amax word).
//   pass 2  every workgroup reduces those maxima and derives the global
//           scale, then each lane loads a block, rotates it, scales and
//           encodes it, and writes 8 code bytes and 1 scale byte.  The
//           rotated tensor never leaves registers.
//
// Arithmetic: binary32, round to nearest even, denormals kept (gfx950
// default), no contraction (-ffp-contract=off); the divisions are the
// compiler's correctly rounded binary32 division or sequences proven equal
// to it.

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cstddef>
#include <cstdlib>
#include <cstdint>
#include <cstring>
#include <tuple>
#include <type_traits>
#include <utility>

#include "nvfp4rq.h"
#include "common.hpp"
#include "pass1.hpp"
#include "pass2.hpp"
#include "mxfp4.hpp"
#include "elementwise.hpp"
#include "calibrate.hpp"

namespace nvfp4rq {
namespace {

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

// Ticks of the device's constant-rate wall clock (the clock wall_clock64
// reads) per millisecond, cached per device; 100 MHz if the runtime does not
// say.
int64_t wall_ticks_per_ms() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 100000;
  int c = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (c == 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeWallClockRate, dev) != hipSuccess || c <= 0)
      c = 100000;  // kHz
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

// Pass 1: 2 workgroups per compute unit, each wave streaming 4 KiB (bf16) per
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

// Pass 2 when it first reduces pass 1's per-workgroup maxima: one 256-block
// chunk per iteration, 8 workgroups per compute unit (the occupancy the
// kernel's 64 registers allow), or 12 for bf16 inputs of at least 96 chunks
// per compute unit, which then run in one and a half waves of workgroups
// (16384 x 8192, step: 93.8-93.9 us with 12 per CU against 97.9-98.0 with
// 8, 95.0 with 10 and 95.2 with 14; at 4096 x 4096, 16 chunks per CU, 12 per
// CU cost 1.3 us; fp32 65536 x 1024 within noise from 8 to 14).  With the
// amax as one word, enqueue_quant launches a workgroup per chunk instead.
int quant_grid(int64_t nb, bool bf16) {
  int64_t want = env_int("NVFP4RQ_QUANT_WGS");
  const int64_t cus = device_cus(), nchunks = (nb + kThreads - 1) / kThreads;
  if (!want) want = (bf16 && nchunks >= 96 * cus ? 12 : 8) * cus;
  return clamp_grid(want, nchunks);
}

// Rotation alone: one workgroup per kThreads * kQuarters quarters (16384 x
// 8192 bf16, kernel-only: 121 us against 124 with 8 persistent workgroups
// per CU).
int quarter_grid(int64_t nq) {
  const int64_t per_wg = static_cast<int64_t>(kThreads) * kQuarters;
  return clamp_grid((nq + per_wg - 1) / per_wg, (nq + per_wg - 1) / per_wg);
}

// Decode: one wave per whole slice of kSliceQuarters quarters, then one wave
// for a partial slice at the end.
template <bool ROTATE, typename SRC>
nvfp4_status launch_decode(const uint8_t* q, const uint8_t* s, const float* gscale, int64_t nq,
                           float* y, SRC src, hipStream_t st) {
  const int64_t per_wg = (kThreads / 64) * kSliceQuarters;
  const int64_t whole = nq / kSliceQuarters;
  if (whole > 0 && launch(decode_kernel<SRC, ROTATE, false>,
                          dim3(clamp_grid((nq + per_wg - 1) / per_wg, (nq + per_wg - 1) / per_wg)),
                          dim3(kThreads), st, q, s, gscale, nq, y, src) != hipSuccess)
    return NVFP4_ERR_HIP;
  if (nq % kSliceQuarters != 0 &&
      launch(decode_kernel<SRC, ROTATE, true>, dim3(1), dim3(64), st, q, s, gscale, nq, y, src) !=
          hipSuccess)
    return NVFP4_ERR_HIP;
  return NVFP4_OK;
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
  // the quantize pass counts 256-block chunks in 32 bits
  if (*nb >= (int64_t{1} << 39)) return NVFP4_ERR_SHAPE;
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

// First 16-byte piece of a bf16 input that pass 1 reads with ordinary loads
// (see launch_rotamax).
int64_t bf16_nt_end(int64_t nb) {
  const int64_t keep_mb = env_int("NVFP4RQ_LLC_KEEP_MB");
  const int64_t keep_pieces = (keep_mb ? keep_mb << 20 : kLastLevelKeep) / 16;
  return 2 * nb > keep_pieces ? 2 * nb - keep_pieces : 0;
}

hipError_t launch_rotamax(const uint16_t* x, int64_t nb, int rotate, uint32_t* bits, int partials,
                          hipStream_t st, Counters counters = Counters{nullptr, 0u}) {
  const dim3 grid(amax_grid(nb, true));
  // The quantize pass walks the tensor last-first and finds the part pass 1
  // read last in the 256 MB last-level cache; the part before the last
  // kLastLevelKeep bytes would be evicted before the quantize pass got to it,
  // so pass 1 streams it with non-temporal loads.  Measured at 16384 x 8192
  // (step, keeping 128 / 144 / 160 / 176 MB, two runs each): 96.9 / 96.2 /
  // 95.9 / 96.1 us; streaming less leaves pass 1 slower, streaming more
  // costs pass 2 its cache hits.  At 32768 x 14336 the rule took 12 us off.
  const int64_t nt_end = bf16_nt_end(nb);
  return rotate ? launch(rotamax_bf16_kernel<true>, grid, dim3(kThreads), st, x, nb, bits, partials, counters,
                         nt_end)
                : launch(rotamax_bf16_kernel<false>, grid, dim3(kThreads), st, x, nb, bits, partials, counters,
                         nt_end);
}

hipError_t launch_rotamax(const float* x, int64_t nb, int rotate, uint32_t* bits, int partials,
                          hipStream_t st, Counters counters = Counters{nullptr, 0u}) {
  const dim3 grid(amax_grid(nb, false));
  return rotate ? launch(rotamax_f32_kernel<true>, grid, dim3(kThreads), st, x, nb, bits, partials, counters)
                : launch(rotamax_f32_kernel<false>, grid, dim3(kThreads), st, x, nb, bits, partials, counters);
}

template <typename T>
nvfp4_status enqueue_rotamax(const T* x, int64_t nb, int rotate, float* amax, hipStream_t st) {
  uint32_t* bits = reinterpret_cast<uint32_t*>(amax);
  if (launch(zero_word_kernel, dim3(1), dim3(1), st, bits) != hipSuccess) return NVFP4_ERR_HIP;
  if (nb == 0) return NVFP4_OK;
  return launch_rotamax(x, nb, rotate, bits, 0, st) == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

// The quantize pass's head wait gives up after this long (see HeadGuard):
// far beyond any wait a scheduled grid needs (the waiting workgroup starts
// waiting once its own chunks are done, when every other workgroup has long
// counted itself in), short enough that a failure shows within a fraction of
// a second.  NVFP4RQ_HEAD_TIMEOUT_US overrides it (tests).
constexpr int64_t kHeadTimeoutMs = 200;
uint64_t head_ticks() {
  const int64_t us = env_int("NVFP4RQ_HEAD_TIMEOUT_US");
  const int64_t per_ms = wall_ticks_per_ms();
  return static_cast<uint64_t>(us > 0 ? per_ms * us / 1000 : per_ms * kHeadTimeoutMs);
}

// Pass 2.  MODE kWord / kGiven: the amax is the word at amax_src (written by
// pass 1 on the same tensor, or kept from elsewhere).  kHead: amax_src holds
// pass 1's per-workgroup maxima (at the head of q or s), the arrival
// counters are at `counters`, and the kernel writes the maxima's maximum to
// amax_out.
template <typename T, AmaxMode MODE, typename SMAP = RowMajorScales>
nvfp4_status enqueue_quant(const T* x, int64_t nb, int rotate, uint32_t* amax_src, Counters counters,
                           float* amax_out, uint8_t* q, uint8_t* s, float* g, hipStream_t st,
                           SMAP smap = SMAP{}) {
  const int allow_fast = env_int("NVFP4RQ_EXACT_ONLY") ? 0 : 1;
  const int64_t nchunks = smap.chunks(nb);
  dim3 grid(quant_grid(nchunks * kThreads, sizeof(T) == 2));
  if constexpr (MODE != kHead) {
    // Amax given as a word: the workgroup prologue is a single load, and a
    // workgroup per chunk beats 8 persistent ones per CU (16384 x 8192 bf16,
    // cold: 62 against 68 us); with per-workgroup maxima to reduce first,
    // the persistent grid stays ahead.
    grid = dim3(clamp_grid(nchunks, nchunks));
    smap.mirror = 1;
  } else {
    // row-major: workgroup 0 visits both head chunks (head_order), so the
    // grid leaves it two visits; the swizzled head is chunk 0 alone
    if (SMAP::kHeadSwap && grid.x > nchunks - 1) grid.x = static_cast<unsigned>(nchunks - 1);
    if constexpr (std::is_same_v<SMAP, RowMajorScales> && sizeof(T) == 2) {
      // bf16: runs of 4 consecutive chunks per XCD (see RowMajorScales::order).
      // fp32 chunks (16 KiB) do best in plain order: at 65536 x 1024 the step
      // took 91.1 us against 92.7 with runs of 4 or 8.
      smap.xcd_order = nchunks % 32 == 0 && !env_int("NVFP4RQ_PLAIN_ORDER") ? 1 : 0;
    }
  }
  const Launch vis = Launch::make(static_cast<uint32_t>(nchunks), grid.x, allow_fast);
  const uint64_t ticks = head_ticks();
  hipError_t e;
  if constexpr (std::is_same_v<SMAP, SwizzledScales>) {
    // Swizzled chunks are 2048 blocks.  When every chunk can have a
    // 1024-thread workgroup at once (2 per CU at 8 waves per SIMD), such
    // workgroups take a chunk's 128 rows in 2 sub-iterations instead of 8:
    // 128 x 1024 (4 chunks) step 15.7 -> 12.6 us, 4096 x 4096 (512) 20.8 ->
    // 19.8 us; with more chunks than that the 256-thread grid wins (8192 x
    // 4096, 1024 chunks: 30.7 against 34.0 us; 16384 x 4096: 53.2 against
    // 57.4 us).
    const int64_t forced = env_int("NVFP4RQ_SWZ_THREADS");
    if (forced ? forced == 1024 : nchunks <= 2LL * device_cus()) {
      e = rotate ? launch(rotquant_kernel<T, true, SMAP, MODE, 1024>, grid, dim3(1024), st, x, nb, amax_src,
                          counters, amax_out, ticks, q, s, g, smap, vis)
                 : launch(rotquant_kernel<T, false, SMAP, MODE, 1024>, grid, dim3(1024), st, x, nb, amax_src,
                          counters, amax_out, ticks, q, s, g, smap, vis);
      return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
    }
  }
  e = rotate ? launch(rotquant_kernel<T, true, SMAP, MODE>, grid, dim3(kThreads), st, x, nb, amax_src,
                      counters, amax_out, ticks, q, s, g, smap, vis)
             : launch(rotquant_kernel<T, false, SMAP, MODE>, grid, dim3(kThreads), st, x, nb, amax_src,
                      counters, amax_out, ticks, q, s, g, smap, vis);
  return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

bool zeroed_word_path(int g1, bool large) {
  return g1 > kMaxPartials || large || env_int("NVFP4RQ_ZEROED_AMAX");
}

// Where pass 1 can leave its per-workgroup maxima and the arrival counters
// (partials null: nowhere).  Row-major scales: the first kHeadBytes of q_out,
// chunks 0 and 1 of the codes (from 512 blocks up).  Swizzled scales: the
// maxima in the first 2 KiB of s_out, chunk 0's four scale tiles, and the
// counters at the start of code rows 0 .. 15, chunk 0's code lines, one
// 128-byte line each (from 16 rows and 16 blocks per row up).
struct Head {
  uint32_t* partials;
  Counters counters;
};
Head head_of(uint8_t* q, uint8_t*, int64_t nb, RowMajorScales) {
  if (kHeadBytes > 8 * nb) return Head{nullptr, Counters{nullptr, 0u}};
  uint32_t* w = reinterpret_cast<uint32_t*>(q);
  return Head{w, Counters{w + kCounterBase, static_cast<uint32_t>(kCounterStride)}};
}
Head head_of(uint8_t* q, uint8_t* s, int64_t, const SwizzledScales& sm) {
  if (sm.rows < kCounters || sm.cb < 16) return Head{nullptr, Counters{nullptr, 0u}};
  return Head{reinterpret_cast<uint32_t*>(s), Counters{reinterpret_cast<uint32_t*>(q), 2 * sm.cb}};
}

// Both passes.  When the head has room (see head_of) and pass 1
// has at most kMaxPartials workgroups, pass 1 leaves per-workgroup maxima
// and cleared counters there (which one pass-2 workgroup overwrites last), so
// no word has to be zeroed first; other tensors and wider pass-1 grids take
// the zeroed-word path.  So do row-major inputs of kOneShotInputBytes and
// more: with the amax in one word, pass 2 runs a workgroup per chunk, which
// streams inputs well past the last-level cache faster than the persistent
// grid that the per-workgroup maxima call for (bf16, 14336 columns, step with
// the zeroing kernel included: 470 MB input even, 587 MB 2.5% faster, 705 MB
// 3.3%, 939 MB 5.5%; below about 470 MB the persistent grid's cache reuse
// wins, 268 MB by 7%).
template <typename T, typename SMAP = RowMajorScales>
nvfp4_status enqueue_both(const T* x, int64_t nb, int rotate, uint8_t* q, uint8_t* s, float* g,
                          float* amax, hipStream_t st, SMAP smap = SMAP{}) {
  const int g1 = amax_grid_for(x, nb);
  // (the swizzled-scale pass gains nothing from it: 368.8 against 366.9 us
  // per step at 939 MB)
  const bool large = std::is_same_v<SMAP, RowMajorScales> &&
                     nb * 16 * static_cast<int64_t>(sizeof(T)) >= kOneShotInputBytes;
  const Head head = head_of(q, s, nb, smap);
  if (nb == 0 || !head.partials || zeroed_word_path(g1, large)) {
    nvfp4_status r = enqueue_rotamax(x, nb, rotate, amax, st);
    if (r != NVFP4_OK) return r;
    return enqueue_quant<T, kWord>(x, nb, rotate, reinterpret_cast<uint32_t*>(amax), Counters{nullptr, 0u},
                                   amax, q, s, g, st, smap);
  }
  if (launch_rotamax(x, nb, rotate, head.partials, 1, st, head.counters) != hipSuccess) return NVFP4_ERR_HIP;
  return enqueue_quant<T, kHead>(x, nb, rotate, head.partials, head.counters, amax, q, s, g, st, smap);
}

// Measurement support (calibrate.hpp): the fused call's launch sequence for
// row-major scales, with the twins in place of the two passes.
hipError_t launch_stream_read(const uint16_t* x, int64_t nb, uint32_t* out, int partials,
                              hipStream_t st, Counters counters) {
  return launch(stream_read_bf16_kernel, dim3(amax_grid(nb, true)), dim3(kThreads), st, x, nb, out,
                partials, counters, bf16_nt_end(nb));
}
hipError_t launch_stream_read(const float* x, int64_t nb, uint32_t* out, int partials,
                              hipStream_t st, Counters counters) {
  return launch(stream_read_f32_kernel, dim3(amax_grid(nb, false)), dim3(kThreads), st, x, nb, out,
                partials, counters);
}

template <typename T>
nvfp4_status check_calibrate(const T* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s, int64_t* nb) {
  nvfp4_status r = check_shape(rows, cols, nb);
  if (r != NVFP4_OK) return r;
  const int64_t n = rows * cols;
  if (n != 0 && (!x || !q || !s)) return NVFP4_ERR_NULL;
  if (n != 0 && (!aligned(x, 16) || !aligned(q, 16))) return NVFP4_ERR_ALIGN;
  const Range rx = range_of(x, n * static_cast<int64_t>(sizeof(T)));
  const Range rq = range_of(q, n / 2), rs = range_of(s, n / 16);
  if (overlap(rx, rq) || overlap(rx, rs) || overlap(rq, rs)) return NVFP4_ERR_ARG;
  return NVFP4_OK;
}

template <typename T>
nvfp4_status stream_calibrate(const T* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s,
                              hipStream_t st) {
  int64_t nb = 0;
  const nvfp4_status r = check_calibrate(x, rows, cols, q, s, &nb);
  if (r != NVFP4_OK) return r;
  if (nb == 0) return NVFP4_OK;
  const int g1 = amax_grid_for(x, nb);
  const bool large = nb * 16 * static_cast<int64_t>(sizeof(T)) >= kOneShotInputBytes;
  RowMajorScales smap{};
  const Head head = head_of(q, s, nb, smap);
  const bool word_path = !head.partials || zeroed_word_path(g1, large);
  uint32_t* word = reinterpret_cast<uint32_t*>(q);
  const int64_t nchunks = smap.chunks(nb);
  dim3 grid(quant_grid(nchunks * kThreads, sizeof(T) == 2));
  if (word_path) {
    if (launch(zero_word_kernel, dim3(1), dim3(1), st, word) != hipSuccess) return NVFP4_ERR_HIP;
    if (launch_stream_read(x, nb, word, 0, st, Counters{nullptr, 0u}) != hipSuccess) return NVFP4_ERR_HIP;
    grid = dim3(clamp_grid(nchunks, nchunks));
    smap.mirror = 1;
  } else {
    if (launch_stream_read(x, nb, word, 1, st, head.counters) != hipSuccess) return NVFP4_ERR_HIP;
    if constexpr (sizeof(T) == 2)
      smap.xcd_order = nchunks % 32 == 0 && !env_int("NVFP4RQ_PLAIN_ORDER") ? 1 : 0;
  }
  if (!word_path && grid.x > nchunks - 1) grid.x = static_cast<unsigned>(nchunks - 1);
  const Launch vis = Launch::make(static_cast<uint32_t>(nchunks), grid.x);
  return launch(stream_rw_kernel<T>, grid, dim3(kThreads), st, x, nb, q, s, smap, vis) == hipSuccess
             ? NVFP4_OK
             : NVFP4_ERR_HIP;
}

// The twin of a single pass with the amax as one word (the given-scale pass,
// MXFP4): one launch, a workgroup per chunk, chunks in reverse index order.
template <typename T>
nvfp4_status stream_calibrate_single(const T* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s,
                                     hipStream_t st) {
  int64_t nb = 0;
  const nvfp4_status r = check_calibrate(x, rows, cols, q, s, &nb);
  if (r != NVFP4_OK) return r;
  if (nb == 0) return NVFP4_OK;
  RowMajorScales smap{};
  smap.mirror = 1;
  const int64_t nchunks = smap.chunks(nb);
  const dim3 grid(clamp_grid(nchunks, nchunks));
  const Launch vis = Launch::make(static_cast<uint32_t>(nchunks), grid.x);
  return launch(stream_rw_kernel<T>, grid, dim3(kThreads), st, x, nb, q, s, smap, vis) == hipSuccess
             ? NVFP4_OK
             : NVFP4_ERR_HIP;
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
  // 128 rows of input (a row tile) are addressed with 32-bit offsets
  if (cols >= (int64_t{1} << 31) / (128 * static_cast<int64_t>(sizeof(T)))) return NVFP4_ERR_SHAPE;
  int64_t nb = 0;
  nvfp4_status r = validate_quant(x, rows, cols, rotate, q, s, g, amax, &nb, false, sbytes);
  if (r != NVFP4_OK) return r;
  const uint32_t cb = static_cast<uint32_t>(cols / 16), ctiles = (cb + 3) / 4;
  SwizzledScales sm{rows, cb, ctiles, (cb + 15) / 16};
  sm.runs16 = sm.cs % 16 == 0 && sm.chunks(nb) % 128 == 0 ? 1 : 0;
  return enqueue_both(x, nb, rotate, q, s, g, amax, st, sm);
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
  // the amax word is only read (the kernel writes through amax_src on the
  // per-workgroup-maxima path alone)
  return enqueue_quant<T, kGiven>(x, nb, rotate,
                                  const_cast<uint32_t*>(reinterpret_cast<const uint32_t*>(amax)),
                                  Counters{nullptr, 0u}, nullptr, q, s, g, st);
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
  // a workgroup per 256 blocks (16384 x 8192 bf16, cold: 58 us against 62
  // with 8 persistent workgroups per CU)
  const dim3 grid(clamp_grid((nb32 + kThreads - 1) / kThreads, (nb32 + kThreads - 1) / kThreads));
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

template <typename T>
nvfp4_status rotate_matrix(const T* x, int64_t rows, int64_t cols, const float* r, float* y,
                           hipStream_t st) {
  int64_t nb = 0;
  nvfp4_status s = check_shape(rows, cols, &nb);
  if (s != NVFP4_OK) return s;
  const int64_t n = rows * cols;
  if ((n != 0 && (!x || !y)) || !r) return NVFP4_ERR_NULL;
  if ((n != 0 && (!aligned(x, 16) || !aligned(y, 16))) || !aligned(r, 16)) return NVFP4_ERR_ALIGN;
  const Range ry = range_of(y, n * 4);
  if (overlap(range_of(x, n * static_cast<int64_t>(sizeof(T))), ry) || overlap(range_of(r, 1024), ry))
    return NVFP4_ERR_ARG;
  if (nb == 0) return NVFP4_OK;
  const int64_t nq = 4 * nb;
  return launch(rotate_matrix_kernel<T>, dim3(quarter_grid(nq)), dim3(kThreads), st, x, nq, r, y) ==
                 hipSuccess
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
  return rotate ? launch_decode<true>(q, s, gscale, nq, y_out, Nvfp4Scales<SMAP>{smap}, stream)
                : launch_decode<false>(q, s, gscale, nq, y_out, Nvfp4Scales<SMAP>{smap}, stream);
}

// The fused call with the timing hook armed for this thread (see launch_impl).
template <typename T>
nvfp4_status timed(const T* x, int64_t rows, int64_t cols, int rotate, uint8_t* q, uint8_t* s,
                   float* g, float* amax, hipStream_t st, hipEvent_t* events, int npairs,
                   int* nkernels) {
  if (!events || npairs < 1 || !nkernels) return NVFP4_ERR_NULL;
  t_events = events;
  t_pairs = npairs;
  t_launched = 0;
  const nvfp4_status r = rotquant(x, rows, cols, rotate, q, s, g, amax, st);
  *nkernels = t_launched;
  t_events = nullptr;
  t_pairs = 0;
  t_launched = 0;
  return r;
}

}  // namespace
}  // namespace nvfp4rq

using namespace nvfp4rq;

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
  return timed(x_bf16, rows, cols, rotate, q_out, s_out, gscale_out, amax_out, stream, events, npairs,
               nkernels);
}

nvfp4_status nvfp4_rotquant_f32_timed(const float* x, int64_t rows, int64_t cols, int rotate,
                                      uint8_t* q_out, uint8_t* s_out, float* gscale_out,
                                      float* amax_out, hipStream_t stream, hipEvent_t* events,
                                      int npairs, int* nkernels) {
  return timed(x, rows, cols, rotate, q_out, s_out, gscale_out, amax_out, stream, events, npairs,
               nkernels);
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
  const float* no_gscale = nullptr;
  return rotate ? launch_decode<true>(q, s, no_gscale, nq, y_out, Mxfp4Scales{}, stream)
                : launch_decode<false>(q, s, no_gscale, nq, y_out, Mxfp4Scales{}, stream);
}

nvfp4_status nvfp4_rotate_matrix(const uint16_t* x_bf16, int64_t rows, int64_t cols, const float* r16,
                                 float* y_out, hipStream_t stream) {
  return rotate_matrix(x_bf16, rows, cols, r16, y_out, stream);
}

nvfp4_status nvfp4_rotate_matrix_f32(const float* x, int64_t rows, int64_t cols, const float* r16,
                                     float* y_out, hipStream_t stream) {
  return rotate_matrix(x, rows, cols, r16, y_out, stream);
}

nvfp4_status nvfp4_stream_calibrate(const uint16_t* x_bf16, int64_t rows, int64_t cols,
                                    uint8_t* q_out, uint8_t* s_out, hipStream_t stream) {
  return stream_calibrate(x_bf16, rows, cols, q_out, s_out, stream);
}

nvfp4_status nvfp4_stream_calibrate_f32(const float* x, int64_t rows, int64_t cols, uint8_t* q_out,
                                        uint8_t* s_out, hipStream_t stream) {
  return stream_calibrate(x, rows, cols, q_out, s_out, stream);
}

nvfp4_status nvfp4_stream_calibrate_single(const uint16_t* x_bf16, int64_t rows, int64_t cols,
                                           uint8_t* q_out, uint8_t* s_out, hipStream_t stream) {
  return stream_calibrate_single(x_bf16, rows, cols, q_out, s_out, stream);
}

nvfp4_status nvfp4_stream_calibrate_single_f32(const float* x, int64_t rows, int64_t cols, uint8_t* q_out,
                                               uint8_t* s_out, hipStream_t stream) {
  return stream_calibrate_single(x, rows, cols, q_out, s_out, stream);
}

const char* nvfp4_status_string(nvfp4_status status) {
  // A C caller may pass any int.  Its bytes are read as an int: loading a value
  // outside the enumerators' range through the C++ enum type is undefined.
  static_assert(sizeof(nvfp4_status) == sizeof(int), "enum size");
  int code = 0;
  std::memcpy(&code, &status, sizeof code);
  switch (code) {
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
