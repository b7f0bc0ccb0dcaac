// cache.hip -- an HBM cache of the hottest rows of host-resident tables.
// "Conditional Memory via Scalable Lookup", section 2.5: n-gram frequencies follow a
// Zipf law, so a small set of rows serves most lookups; keeping those in a faster
// tier (here HBM, in front of the pinned host tables of Figure 2(b)) cuts the
// traffic of the prefetch over PCIe.
//
//   engram_cache_select         host: per table, the `capacity` rows that occur most
//                               often in a sample of indices (ties: smaller row first);
//   engram_cache_build          host + device: an open-addressing hash table per table
//                               mapping row -> cache slot, and the cached rows copied
//                               from the host tables into HBM;
//   engram_prefetch_host_cached the prefetch: one lookup per (token, table); a hit reads
//                               the row from HBM, a miss reads it over PCIe.  The staged
//                               rows are bit-identical to engram_gather's.
//
// Hash table: `slots` entries per table (a power of two, more than `capacity`), each
// {row, cache slot} or {-1, -1}; the home entry of row r is the top log2(slots) bits
// of r * 0x9E3779B1 (Fibonacci hashing), collisions probe linearly.
#include <algorithm>
#include <vector>

#include <string.h>

#include "engram_internal.h"

namespace engram {
namespace {

constexpr uint32_t kFib = 0x9E3779B1u;

__host__ __device__ __forceinline__ uint32_t home_slot(int32_t row, int log2_slots) {
  return ((uint32_t)row * kFib) >> (32 - log2_slots);
}

int log2_exact(int32_t x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return (1 << l) == x ? l : -1;
}

// The gather kernel's layout (threadIdx.x = 16-byte chunk of the concatenated row,
// threadIdx.y = token), one token per thread so every PCIe read of a step is issued
// at once; each lane first looks its (token, table) row up in the cache.
__global__ __launch_bounds__(1024) void prefetch_cached_kernel(const GatherArgs a, const int2* __restrict__ table,
                                                               int log2_slots, const char* __restrict__ cache_rows,
                                                               int32_t* hits) {
  const int c = threadIdx.x;
  const int cpr = a.chunks_per_row;
  const int b = c / cpr;
  const int k = c - b * cpr;
  const int nt = a.n_tables;
  const int64_t row_bytes = (int64_t)cpr * 16;
  const int64_t out_row_bytes = row_bytes * nt;
  const int64_t t = (int64_t)blockIdx.x * blockDim.y + threadIdx.y;
  if (t >= a.n_tok) return;
  const int64_t r = a.idx[t * nt + b];
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  int bad = 0, hit = 0;
  if ((uint64_t)r < (uint64_t)a.rows[b]) {
    const int2* tb = table + ((int64_t)b << log2_slots);
    const uint32_t mask = (1u << log2_slots) - 1u;
    uint32_t s = home_slot((int32_t)r, log2_slots);
    int2 e = tb[s];
    // a table built with these slots always has empty entries; the bound keeps a table
    // of fewer slots than the caller claims from looping forever (it reads as a miss)
    for (uint32_t probes = 1; e.x != (int32_t)r && e.x != -1 && probes <= mask; ++probes) {
      s = (s + 1u) & mask;
      e = tb[s];
    }
    if (e.x == (int32_t)r) {
      v = *reinterpret_cast<const uint4*>(cache_rows + ((int64_t)e.y * nt + b) * row_bytes + k * 16);
      hit = (k == 0);
    } else {
      v = *reinterpret_cast<const uint4*>(a.table[b] + r * row_bytes + k * 16);
    }
  } else {
    bad = (k == 0);  // one count per bad (token, table) pair, as the gather counts
  }
  *reinterpret_cast<uint4*>(a.out + t * out_row_bytes + c * 16) = v;
  if (bad != 0 && a.err_count != nullptr) atomicAdd(a.err_count, bad);
  if (hit != 0 && hits != nullptr) atomicAdd(hits, hit);
}

}  // namespace

void launch_prefetch_cached(const GatherArgs& a, const int2* table, int log2_slots, const char* cache_rows,
                            int32_t* hits, hipStream_t s) {
  const int cpt = a.n_tables * a.chunks_per_row;  // <= 1024, checked by the caller
  int ty = 512 / cpt;
  if (ty < 1) ty = 1;
  const int64_t blocks = (a.n_tok + ty - 1) / ty;
  hipLaunchKernelGGL(prefetch_cached_kernel, dim3((unsigned)blocks), dim3(cpt, ty), 0, s, a, table, log2_slots,
                     cache_rows, hits);
}

}  // namespace engram

using namespace engram;

extern "C" {

engram_status engram_cache_select(const int32_t* idx, int64_t n, int32_t n_tables, int32_t capacity,
                                  int32_t* hot) {
  const char* fn = "engram_cache_select";
  if (n < 0 || n_tables <= 0 || n_tables > ENGRAM_MAX_TABLES || capacity <= 0)
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: bad sizes n=%lld n_tables=%d capacity=%d", fn, (long long)n,
                n_tables, capacity);
  if (hot == nullptr || (n > 0 && idx == nullptr)) return fail(ENGRAM_ERR_INVALID_ARG, "%s: null pointer", fn);
  std::vector<int32_t> col;
  std::vector<std::pair<int64_t, int32_t>> runs;  // (-count, row): ascending = most frequent first
  col.reserve((size_t)n);
  for (int b = 0; b < n_tables; ++b) {
    col.clear();
    for (int64_t t = 0; t < n; ++t) {
      const int32_t r = idx[t * n_tables + b];
      if (r >= 0) col.push_back(r);  // negative indices are not rows
    }
    std::sort(col.begin(), col.end());
    runs.clear();
    for (size_t i = 0; i < col.size();) {
      size_t j = i;
      while (j < col.size() && col[j] == col[i]) ++j;
      runs.emplace_back(-(int64_t)(j - i), col[i]);
      i = j;
    }
    const size_t keep = std::min(runs.size(), (size_t)capacity);
    std::partial_sort(runs.begin(), runs.begin() + keep, runs.end());
    int32_t* out = hot + (int64_t)b * capacity;
    for (size_t i = 0; i < (size_t)capacity; ++i) out[i] = i < keep ? runs[i].second : -1;
  }
  return ENGRAM_OK;
}

engram_status engram_cache_build(const void* const* host_tables, const int64_t* rows, int32_t n_tables, int32_t w,
                                 engram_dtype dtype, const int32_t* hot, int32_t capacity, int32_t slots,
                                 void* table, void* cache_rows, hipStream_t stream) {
  const char* fn = "engram_cache_build";
  if (n_tables <= 0 || n_tables > ENGRAM_MAX_TABLES || capacity <= 0)
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: bad n_tables %d or capacity %d", fn, n_tables, capacity);
  const int l2 = log2_exact(slots);
  if (l2 < 1 || l2 > 30 || slots <= capacity)
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: slots %d must be a power of two above capacity %d", fn, slots, capacity);
  if (enum_arg(dtype) != ENGRAM_F32 && enum_arg(dtype) != ENGRAM_BF16)
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: unknown dtype", fn);
  if (w <= 0 || ((int64_t)w * (dtype == ENGRAM_F32 ? 4 : 2)) % 16 != 0)
    return fail(ENGRAM_ERR_UNSUPPORTED, "%s: row bytes must be a positive multiple of 16", fn);
  if (hot == nullptr || rows == nullptr || host_tables == nullptr || table == nullptr || cache_rows == nullptr ||
      ((uintptr_t)table % 8) != 0 || ((uintptr_t)cache_rows % 16) != 0)
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: null or misaligned pointer", fn);
  // the hash tables, built on the host
  std::vector<int2> ent((size_t)n_tables << l2, make_int2(-1, -1));
  const uint32_t mask = (uint32_t)slots - 1u;
  for (int b = 0; b < n_tables; ++b) {
    int2* tb = ent.data() + ((size_t)b << l2);
    for (int32_t j = 0; j < capacity; ++j) {
      const int32_t r = hot[(int64_t)b * capacity + j];
      if (r < 0) continue;
      if ((int64_t)r >= rows[b])
        return fail(ENGRAM_ERR_INVALID_ARG, "%s: hot row %d of table %d is out of range", fn, r, b);
      uint32_t s = home_slot(r, l2);
      while (tb[s].x != -1 && tb[s].x != r) s = (s + 1u) & mask;
      if (tb[s].x == -1) tb[s] = make_int2(r, j);  // a repeated row keeps its first slot
    }
  }
  hipError_t e = hipMemcpyAsync(table, ent.data(), ent.size() * sizeof(int2), hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "engram_cache_build: hipMemcpyAsync(table)");
  // the cached rows: cache slot j of table b holds row hot[b][j] (zeros for -1), read
  // from the host tables by the prefetch kernel, as [capacity][n_tables * w]
  std::vector<int32_t> idx_t((size_t)capacity * n_tables);
  for (int32_t j = 0; j < capacity; ++j)
    for (int b = 0; b < n_tables; ++b) idx_t[(size_t)j * n_tables + b] = hot[(int64_t)b * capacity + j];
  int32_t* idx_d = nullptr;
  e = hipMallocAsync((void**)&idx_d, idx_t.size() * sizeof(int32_t), stream);
  if (e != hipSuccess) return hip_fail(e, "engram_cache_build: hipMallocAsync");
  e = hipMemcpyAsync(idx_d, idx_t.data(), idx_t.size() * sizeof(int32_t), hipMemcpyHostToDevice, stream);
  engram_status st = e == hipSuccess ? ENGRAM_OK : hip_fail(e, "engram_cache_build: hipMemcpyAsync(idx)");
  if (st == ENGRAM_OK)
    st = engram_prefetch_host(idx_d, capacity, n_tables, host_tables, rows, w, dtype, cache_rows, nullptr, stream);
  const hipError_t ef = hipFreeAsync(idx_d, stream);
  // the host vectors must outlive the copies
  const hipError_t es = hipStreamSynchronize(stream);
  if (st != ENGRAM_OK) return st;
  if (ef != hipSuccess) return hip_fail(ef, "engram_cache_build: hipFreeAsync");
  if (es != hipSuccess) return hip_fail(es, "engram_cache_build: hipStreamSynchronize");
  return ENGRAM_OK;
}

}  // extern "C"
