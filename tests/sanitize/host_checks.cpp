// Host-side checks of libengram's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code only (no GPU is used): argument
// validation of every entry point, which must return before any HIP call, and the
// row cache's host-side hot-row selection against a brute force.  Exits non-zero
// on the first mismatch; the sanitizers abort on any memory or UB error.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <vector>

#include "engram.h"

static int g_fail = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      g_fail = 1;                                                      \
    }                                                                  \
  } while (0)

static void* fake(uintptr_t a) { return (void*)a; }  // aligned, never dereferenced

int main() {
  const int32_t orders[2] = {2, 3};
  uint64_t mult[2 * 2 * 3];
  for (int i = 0; i < 12; ++i) mult[i] = 2 * i + 1;
  const uint32_t rows[4] = {7, 7, 7, 7};
  const int64_t rows64[2] = {10, 10};
  const void* tabs[2] = {fake(256), fake(512)};

  // compress
  EXPECT(engram_compress(nullptr, -1, nullptr, 10, nullptr, nullptr, 0) == ENGRAM_ERR_INVALID_ARG);
  EXPECT(strlen(engram_last_error()) > 0);
  EXPECT(engram_compress((const int32_t*)fake(256), 0, (const int32_t*)fake(256), 10, nullptr, nullptr, 0) ==
         ENGRAM_OK);
  // hash
  EXPECT(engram_hash((const int32_t*)fake(256), 1, 10, 5, 6, orders, 2, 2, mult, rows, 0, (int32_t*)fake(256), 0) ==
         ENGRAM_ERR_INVALID_ARG);
  EXPECT(engram_hash((const int32_t*)fake(256), 1, 10, 0, 10, orders, 2, 17, mult, rows, 0, (int32_t*)fake(256),
                     0) == ENGRAM_ERR_INVALID_ARG);
  const uint32_t bad_rows[4] = {7, 0, 7, 7};
  EXPECT(engram_hash((const int32_t*)fake(256), 1, 10, 0, 10, orders, 2, 2, mult, bad_rows, 0,
                     (int32_t*)fake(256), 0) == ENGRAM_ERR_INVALID_ARG);
  EXPECT(engram_hash((const int32_t*)fake(256), 1, 10, 0, 0, orders, 2, 2, mult, rows, 0, (int32_t*)fake(256), 0) ==
         ENGRAM_OK);
  // gather / prefetch
  EXPECT(engram_gather((const int32_t*)fake(256), 4, 2, tabs, rows64, 4, ENGRAM_BF16, fake(1024), nullptr, 0) ==
         ENGRAM_ERR_UNSUPPORTED);
  EXPECT(engram_gather((const int32_t*)fake(256), 4, 33, tabs, rows64, 8, ENGRAM_BF16, fake(1024), nullptr, 0) ==
         ENGRAM_ERR_INVALID_ARG);
  EXPECT(engram_gather((const int32_t*)fake(256), 4, 2, tabs, rows64, 5120, ENGRAM_BF16, fake(1024), nullptr, 0) ==
         ENGRAM_ERR_UNSUPPORTED);
  EXPECT(engram_gather((const int32_t*)fake(256), 0, 2, tabs, rows64, 8, ENGRAM_BF16, fake(1024), nullptr, 0) ==
         ENGRAM_OK);
  EXPECT(engram_prefetch_host((const int32_t*)fake(256), -1, 2, tabs, rows64, 8, ENGRAM_BF16, fake(1024), nullptr,
                              0) == ENGRAM_ERR_INVALID_ARG);
  // lookup
  const int32_t* map = (const int32_t*)fake(256);
  EXPECT(engram_lookup((const int32_t*)fake(256), 1, 10, 0, 10, map, 100, orders, 2, 2, mult, rows, 0, tabs, 4,
                       ENGRAM_BF16, nullptr, nullptr, fake(1024), nullptr, 0) != ENGRAM_OK);
  // gate: sizes, shapes whose offsets would wrap, unknown modes
  const void* one[1] = {fake(4096)};
  void* out1[1] = {fake(4096)};
  auto gate = [&](int64_t n, int dm, int dmod, int nb, float eps, engram_dtype dt, int kn) {
    return engram_gate_forward(fake(4096), n, dm, dmod, nb, one, one, one, one, one, eps, dt, (engram_key_norm)kn,
                               out1, nullptr, nullptr, 0);
  };
  EXPECT(gate(8, 1000, 2560, 1, 1e-6f, ENGRAM_BF16, 0) == ENGRAM_ERR_UNSUPPORTED);
  EXPECT(gate(8, 1280, 2560, 0, 1e-6f, ENGRAM_BF16, 0) == ENGRAM_ERR_INVALID_ARG);
  EXPECT(gate(8, 1280, 2560, 9, 1e-6f, ENGRAM_BF16, 0) == ENGRAM_ERR_INVALID_ARG);
  EXPECT(gate(8, 1280, 2560, 1, -1.f, ENGRAM_BF16, 0) == ENGRAM_ERR_INVALID_ARG);
  EXPECT(gate(8, 1280, 2560, 1, 1e-6f, ENGRAM_BF16, 2) == ENGRAM_ERR_INVALID_ARG);
  EXPECT(gate(8, 65536, 65536, 1, 1e-6f, ENGRAM_BF16, 0) == ENGRAM_ERR_UNSUPPORTED);
  EXPECT(gate(((int64_t)1 << 31) - 1, 64, 1 << 16, 8, 1e-6f, ENGRAM_BF16, 0) == ENGRAM_ERR_UNSUPPORTED);
  EXPECT(gate((int64_t)1 << 31, 64, 64, 1, 1e-6f, ENGRAM_BF16, 0) == ENGRAM_ERR_UNSUPPORTED);
  EXPECT(gate(0, 1280, 2560, 1, 1e-6f, ENGRAM_BF16, 0) == ENGRAM_OK);
  // lookup and gate in one call: the lookup's and the gate's checks, and rows under 64 values
  const void* tabs4[4] = {fake(256), fake(512), fake(768), fake(1024)};  // one per (order, head)
  auto lookup_gate = [&](int w, int dmod, int nb, int kn) {
    return engram_lookup_gate((const int32_t*)fake(256), 1, 10, 0, 10, map, 100, orders, 2, 2, mult, rows, 0, tabs4,
                              w, dmod, nb, one, one, one, one, one, 1e-6f, (engram_key_norm)kn, out1, nullptr,
                              nullptr, nullptr, nullptr, 0);
  };
  EXPECT(lookup_gate(32, 2560, 1, 0) == ENGRAM_ERR_UNSUPPORTED);
  EXPECT(lookup_gate(12, 2560, 1, 0) == ENGRAM_ERR_UNSUPPORTED);
  EXPECT(lookup_gate(80, 2500, 1, 0) == ENGRAM_ERR_UNSUPPORTED);
  EXPECT(lookup_gate(80, 2560, 0, 0) == ENGRAM_ERR_INVALID_ARG);
  EXPECT(lookup_gate(80, 2560, 1, 7) == ENGRAM_ERR_INVALID_ARG);
  EXPECT(engram_gate_wait_timeouts(nullptr, 0) == ENGRAM_ERR_INVALID_ARG);
  // convolution
  EXPECT(engram_conv_forward(fake(256), 1, 10, 2560, fake(256), fake(256), 9, 3, 1e-6f, ENGRAM_BF16, fake(4096), 0) ==
         ENGRAM_ERR_UNSUPPORTED);
  EXPECT(engram_conv_forward(fake(4096), 1, 10, 64, fake(256), fake(256), 4, 3, 1e-6f, ENGRAM_BF16, fake(4096), 0) ==
         ENGRAM_ERR_INVALID_ARG);  // out overlaps value
  // quantization
  EXPECT(engram_quantize_fp8(fake(256), 4, 10, ENGRAM_BF16, (uint8_t*)fake(256), (float*)fake(256), nullptr, 0) ==
         ENGRAM_ERR_UNSUPPORTED);
  // host allocation arguments
  EXPECT(engram_host_alloc(16, nullptr) == ENGRAM_ERR_INVALID_ARG);
  void* p = fake(16);
  EXPECT(engram_host_alloc(0, &p) == ENGRAM_ERR_INVALID_ARG && p == nullptr);

  // row cache: hot-row selection against a brute force (per column: most frequent
  // first, ties to the smaller row, -1 padding)
  const int n = 5000, nt = 3, cap = 40;
  std::vector<int32_t> idx((size_t)n * nt);
  uint64_t s = 12345;
  for (auto& v : idx) {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    const uint32_t u = (uint32_t)(s >> 33);
    v = (int32_t)((u % 97) * (u % 7) % 300) - ((u % 53) == 0 ? 400 : 0);  // some negative (ignored)
  }
  std::vector<int32_t> hot((size_t)nt * cap, 7);
  EXPECT(engram_cache_select(idx.data(), n, nt, cap, hot.data()) == ENGRAM_OK);
  for (int b = 0; b < nt; ++b) {
    std::map<int32_t, int64_t> cnt;
    for (int t = 0; t < n; ++t)
      if (idx[(size_t)t * nt + b] >= 0) cnt[idx[(size_t)t * nt + b]]++;
    std::vector<std::pair<int64_t, int32_t>> v;
    for (auto& kv : cnt) v.emplace_back(-kv.second, kv.first);
    std::sort(v.begin(), v.end());
    for (int j = 0; j < cap; ++j) EXPECT(hot[(size_t)b * cap + j] == (j < (int)v.size() ? v[j].second : -1));
  }
  EXPECT(engram_cache_select(idx.data(), n, 0, cap, hot.data()) == ENGRAM_ERR_INVALID_ARG);
  EXPECT(engram_cache_build(tabs, rows64, 2, 80, ENGRAM_BF16, hot.data(), 40, 48, fake(256), fake(256), 0) ==
         ENGRAM_ERR_INVALID_ARG);  // slots not a power of two

  if (g_fail) return 1;
  printf("host checks passed\n");
  return 0;
}
