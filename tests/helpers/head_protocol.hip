// Host-side check of the indexing rules the quantize pass's head protocol
// rests on, evaluated with the kernels' own index functions (common.hpp,
// pass2.hpp) for many chunk counts and grid sizes:
//   - the chunk order (with the head's swap, head_order) is a permutation:
//     every chunk is visited, and written, exactly once;
//   - row-major: workgroup 0 visits chunk 1 second-to-last and chunk 0 last,
//     so it writes both head chunks, after all of its other work and after
//     its wait, and no other workgroup writes either; swizzled: workgroup 0
//     visits chunk 0, the whole head, last;
//   - no workgroup gets more chunks than under the plain order;
//   - the head is where the host puts it: row-major, the first 4 KiB of the
//     codes (chunks 0 and 1); swizzled, the maxima in the first 2 KiB of the
//     scales (chunk 0's four tiles) and the counters at the start of code
//     rows 0..15 (chunk 0's code lines), each on its own 128-byte line;
//   - the amax pass's workgroup remap is a bijection on its grid.
// Test code: built and run by tests/test_head_protocol_cpu.py.  Runs on the
// host only; no GPU call is made.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "common.hpp"
#include "pass2.hpp"

using namespace nvfp4rq;

static int failures = 0;
#define CHECK(cond, ...)                                 \
  do {                                                   \
    if (!(cond)) {                                       \
      if (failures < 20) {                               \
        std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
        std::printf(__VA_ARGS__);                        \
        std::printf("\n");                               \
      }                                                  \
      ++failures;                                        \
    }                                                    \
  } while (0)

// Walks every workgroup's visits last-first, as the kernel does.
template <typename SMAP>
static void check_order(const char* tag, const SMAP& smap, uint32_t nchunks, uint32_t grid, bool head) {
  if (head && SMAP::kHeadSwap && grid > nchunks - 1) grid = nchunks - 1;  // as the host launches it
  std::vector<int> visits(nchunks, 0), writer(nchunks, -1);
  const Launch vis = Launch::make(nchunks, grid);
  for (uint32_t wg = 0; wg < grid; ++wg) {
    const uint32_t mine = vis.of(wg);
    CHECK(mine == chunks_of(wg, grid, nchunks), "%s: visit count of wg %u", tag, wg);
    for (int32_t it = static_cast<int32_t>(mine) - 1; it >= 0; --it) {
      const uint32_t i = static_cast<uint32_t>(it) * grid + wg;
      CHECK(i < nchunks, "%s: visit index %u >= %u", tag, i, nchunks);
      const uint32_t c = head_order(smap, i, nchunks, grid, head);
      CHECK(c < nchunks, "%s: chunk %u >= %u (wg %u)", tag, c, nchunks, wg);
      if (c >= nchunks) continue;
      ++visits[c];
      writer[c] = static_cast<int>(wg);
      if (head && c == 0) CHECK(wg == 0 && it == 0, "%s: chunk 0 at wg %u it %d", tag, wg, it);
      if (head && SMAP::kHeadSwap && c == 1) CHECK(wg == 0 && it == 1, "%s: chunk 1 at wg %u it %d", tag, wg, it);
    }
  }
  for (uint32_t c = 0; c < nchunks; ++c)
    CHECK(visits[c] == 1, "%s: chunk %u visited %d times (nchunks %u, grid %u)", tag, c, visits[c], nchunks,
          grid);
  if (head) CHECK(writer[0] == 0, "%s: chunk 0 written by %d", tag, writer[0]);
  if (head && SMAP::kHeadSwap) CHECK(writer[1] == 0, "%s: chunk 1 written by %d", tag, writer[1]);
}

static void check_pass1_remap(int64_t grid) {
  std::vector<int> seen(grid, 0);
  for (int64_t b = 0; b < grid; ++b) {
    const int64_t w = pass1_wg_of(b, grid);
    CHECK(w >= 0 && w < grid, "pass1 grid %lld: wg %lld -> %lld", (long long)grid, (long long)b, (long long)w);
    if (w >= 0 && w < grid) ++seen[w];
  }
  for (int64_t w = 0; w < grid; ++w) CHECK(seen[w] == 1, "pass1 grid %lld: logical %lld hit %d times",
                                           (long long)grid, (long long)w, seen[w]);
}

// Quantize grids the library launches: 8 workgroups per CU for a few CU
// counts, clamped to the chunk count, and the overrides the GPU tests use.
static std::vector<uint32_t> quant_grids(uint32_t nchunks) {
  std::vector<uint32_t> g;
  for (uint32_t want : {8u * 256u, 8u * 304u, 8u * 80u, 8u, 1u, 3u, 5u, 7u, 64u, 1536u, 2048u, 3072u, 100000u})
    g.push_back(want < nchunks ? want : nchunks);
  return g;
}

int main() {
  // pass 1: grids of 2 workgroups per CU for several CU counts, the grids the
  // GPU tests force, and every grid up to 1100
  for (int64_t grid = 1; grid <= 1100; ++grid) check_pass1_remap(grid);
  check_pass1_remap(2 * 304);
  check_pass1_remap(4096);

  // row-major: chunk counts of the workloads and of the tests' shapes, plus
  // a sweep; xcd_order is allowed when the count is a multiple of 32
  std::vector<uint32_t> counts = {2, 3, 4, 31, 32, 33, 63, 64, 96, 128, 255, 256, 4096, 16384, 32768,
                                  4096 * 14 / 16, 524288, 1835008, 262144, 131072, 12300};
  for (uint32_t n = 2; n <= 700; ++n) counts.push_back(n);
  for (uint32_t nchunks : counts) {
    for (uint32_t grid : quant_grids(nchunks)) {
      for (int xo = 0; xo < 2; ++xo) {
        if (xo && nchunks % 32 != 0) continue;
        RowMajorScales rm{xo, 0};
        check_order("row-major", rm, nchunks, grid, true);
      }
    }
    RowMajorScales one{0, 1};  // one-shot grid, amax as a word: no head
    check_order("row-major one-shot", one, nchunks, nchunks, false);
  }
  // the head is the first 4 KiB of q: chunk 0 (2 KiB of codes) holds the
  // kMaxPartials maxima, chunk 1 the counters
  CHECK(kMaxPartials * 4 == kThreads * 8, "maxima fill chunk 0");
  CHECK(4 * (kCounterBase + (kCounters - 1) * kCounterStride) + 4 <= kHeadBytes && kHeadBytes == 2 * kThreads * 8,
        "counters inside chunk 1");

  // swizzled: shapes (rows, cols) and the host's head and runs16 rules
  const int64_t shapes[][2] = {{128, 512},   {128, 1024},  {300, 4112},  {777, 2064}, {4096, 4096},
                               {16384, 8192}, {32768, 14336}, {65536, 1024}, {1, 464},   {129, 480},
                               {256, 8192},  {1000, 1040},  {2048, 4096}, {7, 16384}, {640, 2048}};
  for (auto& sh : shapes) {
    const int64_t rows = sh[0], cols = sh[1];
    const uint32_t cb = static_cast<uint32_t>(cols / 16), ctiles = (cb + 3) / 4, cs = (cb + 15) / 16;
    SwizzledScales sm{rows, cb, ctiles, cs, 0, 0};
    const uint32_t nchunks = sm.chunks(rows * cb);
    const bool head = rows >= kCounters && cb >= 16;  // the host's rule (head_of)
    if (head) {
      // the maxima: chunk 0's tiles are the first 2 KiB of the scales
      int64_t b0;
      int t0;
      sm.chunk_tiles(sm.split(0), &b0, &t0);
      CHECK(b0 == 0 && t0 == 4, "swizzled %lldx%lld head tiles %lld/%d", (long long)rows, (long long)cols,
            (long long)b0, t0);
      CHECK(kMaxPartials * 4 <= 4 * 512, "maxima fit chunk 0's tiles");
      // the counters: code byte r * 8 cb of row r < 16, which chunk 0 writes
      // (row tile 0, column window 0: code bytes 0..127 of rows 0..127), each
      // on its own 128-byte line
      std::vector<uint32_t> codes(static_cast<size_t>(kCounters) * 2 * cb);  // rows 0..15 of the codes
      const Counters cn{codes.data(), 2 * cb};
      for (uint32_t i = 0; i < kCounters; ++i) {
        const int64_t byte = 4 * (cn.at(i) - codes.data());
        const int64_t row = byte / (8 * cb), col_byte = byte % (8 * cb);
        CHECK(row < 128 && row < rows && col_byte < 128, "counter %u at row %lld byte %lld", i, (long long)row,
              (long long)col_byte);
        CHECK(sm.split(static_cast<uint32_t>(0)).rt == row / 128 && col_byte / 128 == 0,
              "counter %u outside chunk 0", i);
        if (i > 0) CHECK(byte / 128 != 4 * (cn.at(i - 1) - codes.data()) / 128,
                         "counters %u and %u share a line", i - 1, i);
      }
    }
    for (uint32_t grid : quant_grids(nchunks)) {
      for (int r16 = 0; r16 < 2; ++r16) {
        if (r16 && !(cs % 16 == 0 && nchunks % 128 == 0)) continue;
        sm.runs16 = r16;
        sm.mirror = 0;
        check_order("swizzled", sm, nchunks, grid, head);
      }
    }
    sm.runs16 = 0;
    sm.mirror = 1;
    check_order("swizzled one-shot", sm, nchunks, nchunks, false);
  }
  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("head protocol indexing ok\n");
  return 0;
}
