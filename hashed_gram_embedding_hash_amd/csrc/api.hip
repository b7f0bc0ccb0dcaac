// api.hip -- the C ABI of include/engram.h: argument validation, error
// reporting and kernel launches.  Every check happens on the host before
// anything is enqueued, so a non-OK status never leaves partial work behind.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "engram_internal.h"

namespace engram {

static thread_local char g_err[512];

engram_status fail(engram_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

engram_status hip_fail(hipError_t e, const char* what) {
  return fail(ENGRAM_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

engram_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, what);
  return ENGRAM_OK;
}

}  // namespace engram

using namespace engram;

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t dtype_size(int dt) { return dt == ENGRAM_F32 ? 4 : 2; }

bool valid_dtype(int dt) { return dt == ENGRAM_F32 || dt == ENGRAM_BF16; }

bool valid_key_norm(int kn) { return kn == ENGRAM_KEY_NORM_MEMORY || kn == ENGRAM_KEY_NORM_PROJECTED; }

// Shared validation of engram_gather / engram_prefetch_host.
engram_status check_gather(const char* fn, const int32_t* idx, int64_t n_tok, int32_t n_tables,
                           const void* const* tables, const int64_t* rows, int32_t w,
                           int dtype, void* out) {
  if (n_tok < 0) return fail(ENGRAM_ERR_INVALID_ARG, "%s: n_tok < 0", fn);
  if (n_tables <= 0 || n_tables > ENGRAM_MAX_TABLES)
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: n_tables %d not in [1, %d]", fn, n_tables,
                ENGRAM_MAX_TABLES);
  if (!valid_dtype(dtype)) return fail(ENGRAM_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
  if (w <= 0) return fail(ENGRAM_ERR_INVALID_ARG, "%s: w must be positive", fn);
  if (tables == nullptr || rows == nullptr)
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: null tables or rows array", fn);
  const int64_t row_bytes = (int64_t)w * (int64_t)dtype_size(dtype);
  if (row_bytes % 16 != 0)
    return fail(ENGRAM_ERR_UNSUPPORTED, "%s: row bytes %lld not a multiple of 16", fn,
                (long long)row_bytes);
  if ((row_bytes / 16) * n_tables > 1024)
    return fail(ENGRAM_ERR_UNSUPPORTED, "%s: concatenated row of %lld bytes exceeds 16 KiB", fn,
                (long long)(row_bytes * n_tables));
  for (int b = 0; b < n_tables; ++b) {
    if (rows[b] <= 0) return fail(ENGRAM_ERR_INVALID_ARG, "%s: rows[%d] must be positive", fn, b);
    if (tables[b] == nullptr || !aligned(tables[b], 16))
      return fail(ENGRAM_ERR_INVALID_ARG, "%s: table %d null or not 16-byte aligned", fn, b);
  }
  if (n_tok > 0 && (idx == nullptr || out == nullptr || !aligned(out, 16) || !aligned(idx, 4)))
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: null or misaligned idx/out", fn);
  return ENGRAM_OK;
}

// Device address of a pinned host allocation, or nullptr if `p` is not one.
const void* mapped_host_pointer(const void* p) {
  hipPointerAttribute_t attr;
  memset(&attr, 0, sizeof attr);
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky lookup error
    return nullptr;
  }
  if (attr.type != hipMemoryTypeHost || attr.devicePointer == nullptr) return nullptr;
  // devicePointer/hostPointer describe the allocation containing p
  const char* hb = (const char*)attr.hostPointer;
  const char* db = (const char*)attr.devicePointer;
  if (hb == nullptr) return db;
  return db + ((const char*)p - hb);
}

// The library scratch (the bf16 gate's folded key weights, partial sums, gates and
// work-queue counters; the convolution's per-token inverse RMS): one grow-only buffer
// per device, reused by every call.  A call on the stream that used it last needs
// nothing more (stream order); a call on another stream first waits for an event
// recorded after the previous use.  Growing frees the old buffer in stream order behind
// that wait.  The lock is held from acquiring the buffer until the launches and the
// event record are enqueued, so concurrent host threads take turns.  The current buffer
// lives until the process ends; a replaced one is freed behind the growing call, which
// invalidates graphs captured with it.
struct Scratch {
  void* ptr = nullptr;
  size_t bytes = 0;
  hipStream_t last = nullptr;
  hipEvent_t done = nullptr;
  bool used = false;
};
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
Scratch g_scratch[kMaxDevices];

// Runs launch(ptr) with ptr pointing at >= `bytes` of the current device's scratch.
template <class Launch>
engram_status with_scratch(const char* fn, size_t bytes, hipStream_t stream, Launch&& launch) {
  auto hip_fail = [fn](hipError_t e, const char* what) {
    return fail(ENGRAM_ERR_HIP, "%s: %s: %s (%d)", fn, what, hipGetErrorString(e), (int)e);
  };
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(ENGRAM_ERR_UNSUPPORTED, "%s: device %d", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  Scratch& g = g_scratch[dev];
  if (g.done == nullptr) {
    e = hipEventCreateWithFlags(&g.done, hipEventDisableTiming);
    if (e != hipSuccess) {
      g.done = nullptr;
      return hip_fail(e, "hipEventCreateWithFlags(scratch)");
    }
  }
  if (g.used && g.last != stream) {
    e = hipStreamWaitEvent(stream, g.done, 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent(scratch)");
  }
  if (g.bytes < bytes) {
    if (g.ptr != nullptr) {
      e = hipFreeAsync(g.ptr, stream);
      g.ptr = nullptr;
      g.bytes = 0;
      if (e != hipSuccess) return hip_fail(e, "hipFreeAsync(scratch)");
    }
    const size_t grow = bytes + bytes / 4;  // slack for slightly larger later calls
    e = hipMallocAsync(&g.ptr, grow, stream);
    if (e != hipSuccess) {
      g.ptr = nullptr;
      (void)hipGetLastError();  // the failed allocation must not be reported by a later call's launch check
      return hip_fail(e, "hipMallocAsync(scratch)");
    }
    g.bytes = grow;
  }
  launch(g.ptr);
  const engram_status st = check_launch(fn);
  e = hipEventRecord(g.done, stream);
  g.last = stream;
  g.used = true;
  if (st != ENGRAM_OK) return st;
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord(scratch)");
  return ENGRAM_OK;
}

}  // namespace

extern "C" {

const char* engram_last_error(void) { return g_err; }

const char* engram_version(void) { return "engram-mi355x 0.1.0 (gfx950)"; }

engram_status engram_compress(const int32_t* raw, int64_t n, const int32_t* map, int32_t vocab,
                              int32_t* out, int32_t* err_count, hipStream_t stream) {
  if (n < 0) return fail(ENGRAM_ERR_INVALID_ARG, "engram_compress: n < 0");
  if (vocab <= 0) return fail(ENGRAM_ERR_INVALID_ARG, "engram_compress: vocab must be positive");
  if (map == nullptr) return fail(ENGRAM_ERR_INVALID_ARG, "engram_compress: null map");
  if (n == 0) return ENGRAM_OK;
  if (raw == nullptr || out == nullptr)
    return fail(ENGRAM_ERR_INVALID_ARG, "engram_compress: null raw/out");
  launch_compress(raw, n, map, vocab, out, err_count, stream);
  return check_launch("engram_compress");
}

}  // extern "C"

namespace {

// engram_hash, and with `map` set engram_compress_hash
// The hashing arguments, checked and copied into `a`.  *empty: nothing to launch (batch or
// t_count is 0); then the pointers are not checked.  need_idx: idx must be non-null.
engram_status hash_args(const char* fn, const int32_t* ids, int32_t batch, int64_t ld, int64_t t_begin,
                        int64_t t_count, const int32_t* map, int32_t vocab, const int32_t* orders,
                        int32_t n_orders, int32_t heads, const uint64_t* mult, const uint32_t* rows,
                        int32_t pad_id, int32_t* ids_out, int32_t* idx, int32_t* err_count, bool need_idx,
                        HashArgs& a, bool* empty) {
  *empty = false;
  if (batch < 0 || ld < 0 || t_begin < 0 || t_count < 0)
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: negative size", fn);
  if (t_begin + t_count > ld)
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: window [%lld, %lld) exceeds row length %lld", fn,
                (long long)t_begin, (long long)(t_begin + t_count), (long long)ld);
  if (orders == nullptr || mult == nullptr || rows == nullptr)
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: null orders/mult/rows", fn);
  if (n_orders <= 0 || heads <= 0 || (int64_t)n_orders * heads > ENGRAM_MAX_TABLES)
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: n_orders*heads must be in [1, %d]", fn,
                ENGRAM_MAX_TABLES);
  int max_order = 0;
  for (int o = 0; o < n_orders; ++o) {
    if (orders[o] < 1 || orders[o] > ENGRAM_MAX_ORDER)
      return fail(ENGRAM_ERR_INVALID_ARG, "%s: orders[%d] = %d not in [1, %d]", fn, o, orders[o],
                  ENGRAM_MAX_ORDER);
    if (orders[o] > max_order) max_order = orders[o];
  }
  memset(&a, 0, sizeof a);
  const int nt = n_orders * heads;
  for (int o = 0; o < n_orders; ++o) {
    for (int k = 0; k < heads; ++k) {
      const int tb = o * heads + k;
      const uint32_t M = rows[tb];
      if (M == 0 || M >= (1u << 31))
        return fail(ENGRAM_ERR_INVALID_ARG, "%s: rows[%d] = %u not in [1, 2^31)", fn, tb, M);
      a.rows[tb] = M;
      a.barrett[tb] = ~0ull / M;
      a.order[tb] = orders[o];
      for (int j = 0; j < orders[o]; ++j) a.mult[tb][j] = mult[((int64_t)o * heads + k) * max_order + j];
    }
  }
  if (batch == 0 || t_count == 0) {
    *empty = true;
    return ENGRAM_OK;
  }
  if (ids == nullptr || (need_idx && idx == nullptr)) return fail(ENGRAM_ERR_INVALID_ARG, "%s: null ids/idx", fn);
  const uint64_t blocks = (uint64_t)((t_count + 63) / 64) * (uint64_t)batch;
  if (blocks >= (1ull << 31))
    return fail(ENGRAM_ERR_UNSUPPORTED, "%s: %llu workgroups exceed one launch", fn,
                (unsigned long long)blocks);
  a.ids = ids;
  a.idx = idx;
  a.ld = ld;
  a.t_begin = t_begin;
  a.t_count = t_count;
  a.n_tables = nt;
  a.max_order = max_order;
  a.pad_id = pad_id;
  a.map = map;
  a.vocab = vocab;
  a.ids_out = ids_out;
  a.err_count = err_count;
  a.batch = batch;
  return ENGRAM_OK;
}

engram_status hash_impl(const char* fn, const int32_t* ids, int32_t batch, int64_t ld, int64_t t_begin,
                        int64_t t_count, const int32_t* map, int32_t vocab, const int32_t* orders,
                        int32_t n_orders, int32_t heads, const uint64_t* mult, const uint32_t* rows,
                        int32_t pad_id, int32_t* ids_out, int32_t* idx, int32_t* err_count, hipStream_t stream) {
  HashArgs a;
  bool empty = false;
  const engram_status st = hash_args(fn, ids, batch, ld, t_begin, t_count, map, vocab, orders, n_orders, heads,
                                     mult, rows, pad_id, ids_out, idx, err_count, true, a, &empty);
  if (st != ENGRAM_OK || empty) return st;
  launch_hash(a, stream);
  return check_launch(fn);
}

}  // namespace

extern "C" {

engram_status engram_hash(const int32_t* ids, int32_t batch, int64_t ld, int64_t t_begin,
                          int64_t t_count, const int32_t* orders, int32_t n_orders, int32_t heads,
                          const uint64_t* mult, const uint32_t* rows, int32_t pad_id, int32_t* idx,
                          hipStream_t stream) {
  return hash_impl("engram_hash", ids, batch, ld, t_begin, t_count, nullptr, 0, orders, n_orders, heads, mult,
                   rows, pad_id, nullptr, idx, nullptr, stream);
}

engram_status engram_compress_hash(const int32_t* raw, int32_t batch, int64_t ld, int64_t t_begin,
                                   int64_t t_count, const int32_t* map, int32_t vocab, const int32_t* orders,
                                   int32_t n_orders, int32_t heads, const uint64_t* mult, const uint32_t* rows,
                                   int32_t pad_id, int32_t* ids_out, int32_t* idx, int32_t* err_count,
                                   hipStream_t stream) {
  const char* fn = "engram_compress_hash";
  if (map == nullptr) return fail(ENGRAM_ERR_INVALID_ARG, "%s: null map", fn);
  if (vocab <= 0) return fail(ENGRAM_ERR_INVALID_ARG, "%s: vocab must be positive", fn);
  return hash_impl(fn, raw, batch, ld, t_begin, t_count, map, vocab, orders, n_orders, heads, mult, rows, pad_id,
                   ids_out, idx, err_count, stream);
}

engram_status engram_gather(const int32_t* idx, int64_t n_tok, int32_t n_tables,
                            const void* const* tables, const int64_t* rows, int32_t w,
                            engram_dtype dtype, void* out, int32_t* err_count, hipStream_t stream) {
  const engram_status st = check_gather("engram_gather", idx, n_tok, n_tables, tables, rows, w, enum_arg(dtype), out);
  if (st != ENGRAM_OK) return st;
  if (n_tok == 0) return ENGRAM_OK;
  GatherArgs a;
  memset(&a, 0, sizeof a);
  for (int b = 0; b < n_tables; ++b) {
    a.table[b] = (const char*)tables[b];
    a.rows[b] = rows[b];
  }
  a.idx = idx;
  a.out = (char*)out;
  a.err_count = err_count;
  a.n_tok = n_tok;
  a.n_tables = n_tables;
  a.chunks_per_row = (int32_t)(w * dtype_size(dtype) / 16);
  launch_gather(a, false, stream);
  return check_launch("engram_gather");
}

engram_status engram_lookup(const int32_t* raw, int32_t batch, int64_t ld, int64_t t_begin, int64_t t_count,
                            const int32_t* map, int32_t vocab, const int32_t* orders, int32_t n_orders,
                            int32_t heads, const uint64_t* mult, const uint32_t* rows, int32_t pad_id,
                            const void* const* tables, int32_t w, engram_dtype dtype, int32_t* ids_out,
                            int32_t* idx_out, void* out, int32_t* err_count, hipStream_t stream) {
  const char* fn = "engram_lookup";
  HashArgs h;
  bool empty = false;
  engram_status st = hash_args(fn, raw, batch, ld, t_begin, t_count, map, vocab, orders, n_orders, heads, mult,
                               rows, pad_id, ids_out, idx_out, err_count, false, h, &empty);
  if (st != ENGRAM_OK) return st;
  const int nt = n_orders * heads;
  int64_t rows64[ENGRAM_MAX_TABLES];
  for (int b = 0; b < nt; ++b) rows64[b] = rows[b];
  const int64_t n_tok = empty ? 0 : (int64_t)batch * t_count;
  // the gather's checks (idx is not read: a stand-in keeps the null check quiet)
  static const int32_t no_idx = 0;
  st = check_gather(fn, &no_idx, n_tok, nt, tables, rows64, w, enum_arg(dtype), out);
  if (st != ENGRAM_OK || empty) return st;
  if (idx_out != nullptr && !aligned(idx_out, 4)) return fail(ENGRAM_ERR_INVALID_ARG, "%s: misaligned idx_out", fn);
  if ((uint64_t)((t_count + 7) / 8) * (uint64_t)batch >= (1ull << 31))  // at least 8 positions per workgroup
    return fail(ENGRAM_ERR_UNSUPPORTED, "%s: too many positions for one launch", fn);
  GatherArgs g;
  memset(&g, 0, sizeof g);
  for (int b = 0; b < nt; ++b) {
    g.table[b] = (const char*)tables[b];
    g.rows[b] = rows64[b];
  }
  g.out = (char*)out;
  g.n_tok = n_tok;
  g.n_tables = nt;
  g.chunks_per_row = (int32_t)(w * dtype_size(dtype) / 16);
  launch_lookup(h, g, nullptr, stream);
  return check_launch(fn);
}

engram_status engram_lookup_fp8(const int32_t* raw, int32_t batch, int64_t ld, int64_t t_begin, int64_t t_count,
                                const int32_t* map, int32_t vocab, const int32_t* orders, int32_t n_orders,
                                int32_t heads, const uint64_t* mult, const uint32_t* rows, int32_t pad_id,
                                const void* const* tables, int32_t w, int32_t* ids_out, int32_t* idx_out,
                                uint8_t* codes, float* scales, float* sumsq, int32_t* err_count, hipStream_t stream) {
  const char* fn = "engram_lookup_fp8";
  HashArgs h;
  bool empty = false;
  engram_status st = hash_args(fn, raw, batch, ld, t_begin, t_count, map, vocab, orders, n_orders, heads, mult,
                               rows, pad_id, ids_out, idx_out, err_count, false, h, &empty);
  if (st != ENGRAM_OK) return st;
  const int nt = n_orders * heads;
  int64_t rows64[ENGRAM_MAX_TABLES];
  for (int b = 0; b < nt; ++b) rows64[b] = rows[b];
  const int64_t n_tok = empty ? 0 : (int64_t)batch * t_count;
  static const int32_t no_idx = 0;
  // the gather's checks on bf16 rows (codes stands in for the output)
  st = check_gather(fn, &no_idx, n_tok, nt, tables, rows64, w, ENGRAM_BF16, codes);
  if (st != ENGRAM_OK || empty) return st;
  if (scales == nullptr || !aligned(scales, 4) || (sumsq != nullptr && !aligned(sumsq, 4)))
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: null or misaligned scales/sumsq", fn);
  if (idx_out != nullptr && !aligned(idx_out, 4)) return fail(ENGRAM_ERR_INVALID_ARG, "%s: misaligned idx_out", fn);
  if ((uint64_t)((t_count + 7) / 8) * (uint64_t)batch >= (1ull << 31))
    return fail(ENGRAM_ERR_UNSUPPORTED, "%s: too many positions for one launch", fn);
  GatherArgs g;
  memset(&g, 0, sizeof g);
  for (int b = 0; b < nt; ++b) {
    g.table[b] = (const char*)tables[b];
    g.rows[b] = rows64[b];
  }
  g.n_tok = n_tok;
  g.n_tables = nt;
  g.chunks_per_row = (int32_t)(w * 2 / 16);
  const Q8Out q{codes, scales, sumsq};
  launch_lookup(h, g, &q, stream);
  return check_launch(fn);
}

engram_status engram_prefetch_host(const int32_t* idx, int64_t n_tok, int32_t n_tables,
                                   const void* const* host_tables, const int64_t* rows, int32_t w,
                                   engram_dtype dtype, void* staging, int32_t* err_count,
                                   hipStream_t stream) {
  const char* fn = "engram_prefetch_host";
  const engram_status st = check_gather(fn, idx, n_tok, n_tables, host_tables, rows, w, enum_arg(dtype), staging);
  if (st != ENGRAM_OK) return st;
  GatherArgs a;
  memset(&a, 0, sizeof a);
  for (int b = 0; b < n_tables; ++b) {
    const void* d = mapped_host_pointer(host_tables[b]);
    if (d == nullptr)
      return fail(ENGRAM_ERR_INVALID_ARG, "%s: table %d is not pinned, device-mapped host memory", fn, b);
    a.table[b] = (const char*)d;
    a.rows[b] = rows[b];
  }
  if (n_tok == 0) return ENGRAM_OK;
  a.idx = idx;
  a.out = (char*)staging;
  a.err_count = err_count;
  a.n_tok = n_tok;
  a.n_tables = n_tables;
  a.chunks_per_row = (int32_t)(w * dtype_size(dtype) / 16);
  launch_gather(a, true, stream);
  return check_launch(fn);
}

engram_status engram_prefetch_host_cached(const int32_t* idx, int64_t n_tok, int32_t n_tables,
                                          const void* const* host_tables, const int64_t* rows, int32_t w,
                                          engram_dtype dtype, const void* table, int32_t slots,
                                          const void* cache_rows, void* staging, int32_t* hits,
                                          int32_t* err_count, hipStream_t stream) {
  const char* fn = "engram_prefetch_host_cached";
  const engram_status st = check_gather(fn, idx, n_tok, n_tables, host_tables, rows, w, enum_arg(dtype), staging);
  if (st != ENGRAM_OK) return st;
  int l2 = 0;
  while (l2 < 31 && (1 << l2) < slots) ++l2;
  if (slots < 2 || (1 << l2) != slots || l2 > 30)
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: slots %d must be a power of two", fn, slots);
  if (table == nullptr || cache_rows == nullptr || !aligned(table, 8) || !aligned(cache_rows, 16))
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: null or misaligned cache table/rows", fn);
  GatherArgs a;
  memset(&a, 0, sizeof a);
  for (int b = 0; b < n_tables; ++b) {
    const void* d = mapped_host_pointer(host_tables[b]);
    if (d == nullptr)
      return fail(ENGRAM_ERR_INVALID_ARG, "%s: table %d is not pinned, device-mapped host memory", fn, b);
    a.table[b] = (const char*)d;
    a.rows[b] = rows[b];
  }
  if (n_tok == 0) return ENGRAM_OK;
  a.idx = idx;
  a.out = (char*)staging;
  a.err_count = err_count;
  a.n_tok = n_tok;
  a.n_tables = n_tables;
  a.chunks_per_row = (int32_t)(w * dtype_size(dtype) / 16);
  launch_prefetch_cached(a, (const int2*)table, l2, (const char*)cache_rows, hits, stream);
  return check_launch(fn);
}

}  // extern "C"

namespace {

// The arguments of both gate entry points: checked, and copied into `a` (n_tok == 0
// leaves `a` unfilled: nothing to launch).
engram_status gate_args(const char* fn, const void* mem, int64_t n_tok, int32_t d_mem, int32_t d_model,
                        int32_t n_branch, const void* const* h, const void* const* wk, const void* const* wv,
                        const void* const* gq, const void* const* gk, float eps, int dtype,
                        int key_norm, void* const* out, float* gate_out, void* const* value_out,
                        GateArgs& a) {
  if (n_tok < 0 || d_mem <= 0 || d_model <= 0)
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: bad sizes n_tok=%lld d_mem=%d d_model=%d", fn,
                (long long)n_tok, d_mem, d_model);
  if (n_branch <= 0 || n_branch > ENGRAM_MAX_BRANCHES)
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: n_branch %d not in [1, %d]", fn, n_branch,
                ENGRAM_MAX_BRANCHES);
  if (!valid_dtype(dtype)) return fail(ENGRAM_ERR_INVALID_ARG, "%s: unknown dtype", fn);
  if (!(eps >= 0.f)) return fail(ENGRAM_ERR_INVALID_ARG, "%s: eps must be >= 0", fn);
  if (!valid_key_norm(key_norm))
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: unknown key_norm %d", fn, key_norm);
  if (h == nullptr || wk == nullptr || wv == nullptr || gq == nullptr || gk == nullptr || out == nullptr)
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: null pointer array", fn);
  if (dtype == ENGRAM_BF16 && (d_mem % 64 != 0 || d_model % 32 != 0))
    return fail(ENGRAM_ERR_UNSUPPORTED, "%s: bf16 needs d_mem %% 64 == 0 and d_model %% 32 == 0 (got %d, %d)",
                fn, d_mem, d_model);
  if (n_tok > 0x7fffffffLL) return fail(ENGRAM_ERR_UNSUPPORTED, "%s: n_tok >= 2^31", fn);
  if (dtype == ENGRAM_BF16) {
    // the persistent kernel forms weight offsets (row * d_mem + column, in elements or
    // FP8 bytes) in 32 bits and numbers its tiles in int
    if ((int64_t)d_model * (int64_t)d_mem >= (1ll << 32))
      return fail(ENGRAM_ERR_UNSUPPORTED, "%s: d_model * d_mem = %lld >= 2^32", fn,
                  (long long)d_model * (long long)d_mem);
    const int64_t tiles = ((n_tok + 255) / 256) * (int64_t)n_branch * (((int64_t)d_model + 255) / 256);
    if (tiles > (1ll << 29))
      return fail(ENGRAM_ERR_UNSUPPORTED, "%s: %lld tiles of 256 x 256 exceed 2^29 per launch", fn,
                  (long long)tiles);
  }
  const size_t al = dtype == ENGRAM_BF16 ? 16 : 4;
  if (n_tok > 0 && (mem == nullptr || !aligned(mem, al)))
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: null or misaligned mem", fn);
  if (gate_out != nullptr && !aligned(gate_out, 4))
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: misaligned gate_out", fn);
  memset(&a, 0, sizeof a);
  for (int m = 0; m < n_branch; ++m) {
    if (wk[m] == nullptr || wv[m] == nullptr || gq[m] == nullptr || gk[m] == nullptr ||
        !aligned(wk[m], al) || !aligned(wv[m], al) || !aligned(gq[m], al) || !aligned(gk[m], al))
      return fail(ENGRAM_ERR_INVALID_ARG, "%s: branch %d: null or misaligned weights/gains", fn, m);
    if (n_tok > 0 && (h[m] == nullptr || out[m] == nullptr || !aligned(h[m], al) || !aligned(out[m], al)))
      return fail(ENGRAM_ERR_INVALID_ARG, "%s: branch %d: null or misaligned h/out", fn, m);
    a.h[m] = h[m];
    a.wk[m] = wk[m];
    a.wv[m] = wv[m];
    a.gq[m] = gq[m];
    a.gk[m] = gk[m];
    a.out[m] = out[m];
    a.vout[m] = value_out != nullptr ? value_out[m] : nullptr;
    if (n_tok > 0 && a.vout[m] != nullptr && !aligned(a.vout[m], al))
      return fail(ENGRAM_ERR_INVALID_ARG, "%s: branch %d: misaligned value_out", fn, m);
  }
  a.mem = mem;
  a.gate_out = gate_out;
  a.n_tok = n_tok;
  a.d_mem = d_mem;
  a.d_model = d_model;
  a.n_branch = n_branch;
  a.eps = eps;
  a.inv_sqrt_d = 1.0f / sqrtf((float)d_model);
  a.key_norm = (int32_t)key_norm;
  return ENGRAM_OK;
}

}  // namespace

extern "C" {

engram_status engram_gate_forward(const void* mem, int64_t n_tok, int32_t d_mem, int32_t d_model,
                                  int32_t n_branch, const void* const* h, const void* const* wk,
                                  const void* const* wv, const void* const* gq,
                                  const void* const* gk, float eps, engram_dtype dtype,
                                  engram_key_norm key_norm, void* const* out, float* gate_out,
                                  void* const* value_out, hipStream_t stream) {
  const char* fn = "engram_gate_forward";
  GateArgs a;
  const int dt = enum_arg(dtype), kn = enum_arg(key_norm);
  const engram_status st = gate_args(fn, mem, n_tok, d_mem, d_model, n_branch, h, wk, wv, gq, gk, eps, dt, kn, out,
                                     gate_out, value_out, a);
  if (st != ENGRAM_OK || n_tok == 0) return st;

  if (dt == ENGRAM_F32) {
    // the fp32 path stages the normalised memory vector (and the projected key) in fp64
    const size_t lds = (size_t)d_mem * 8 + (kn == ENGRAM_KEY_NORM_PROJECTED ? (size_t)d_model * 8 : 0);
    if (lds > 128 * 1024)
      return fail(ENGRAM_ERR_UNSUPPORTED, "%s: fp32 path needs d_mem (+ d_model for the projected key norm) "
                  "<= 16384", fn);
    launch_gate_f32(a, stream);
    return check_launch(fn);
  }

  const size_t bytes = gate_bf16_scratch_bytes(a, false);
  return with_scratch(fn, bytes, stream, [&](void* p) {
    a.part_dot = (float*)p;
    launch_gate_bf16(a, false, stream);
  });
}

engram_status engram_gate_forward_noalloc(const void* mem, int64_t n_tok, int32_t d_mem, int32_t d_model,
                                          int32_t n_branch, const void* const* h, const void* const* wk,
                                          const void* const* wv, const void* const* gq, const void* const* gk,
                                          float eps, engram_dtype dtype, engram_key_norm key_norm, void* const* out,
                                          float* gate_out, void* const* value_out, hipStream_t stream) {
  const char* fn = "engram_gate_forward_noalloc";
  GateArgs a;
  const int dt = enum_arg(dtype), kn = enum_arg(key_norm);
  const engram_status st = gate_args(fn, mem, n_tok, d_mem, d_model, n_branch, h, wk, wv, gq, gk, eps, dt, kn, out,
                                     gate_out, value_out, a);
  if (st != ENGRAM_OK || n_tok == 0) return st;
  if (dt == ENGRAM_F32) {  // the fp32 path uses no scratch
    const size_t lds = (size_t)d_mem * 8 + (kn == ENGRAM_KEY_NORM_PROJECTED ? (size_t)d_model * 8 : 0);
    if (lds > 128 * 1024)
      return fail(ENGRAM_ERR_UNSUPPORTED, "%s: fp32 path needs d_mem (+ d_model for the projected key norm) "
                  "<= 16384", fn);
    launch_gate_f32(a, stream);
    return check_launch(fn);
  }
  return gate_forward_noalloc(fn, a, stream);
}

engram_status engram_gate_wait_timeouts(int32_t* count, int32_t reset) {
  if (count == nullptr) return fail(ENGRAM_ERR_INVALID_ARG, "engram_gate_wait_timeouts: null count");
  const hipError_t e = gate_wait_timeouts(count, reset != 0);
  if (e != hipSuccess) return hip_fail(e, "engram_gate_wait_timeouts");
  return ENGRAM_OK;
}

engram_status engram_debug_force_gate_timeout(int32_t on) {
  set_gate_forced_wait_timeout(on != 0);
  return ENGRAM_OK;
}

engram_status engram_debug_gate_key_form(int32_t form) {
  if (form < 0 || form > 2) return fail(ENGRAM_ERR_INVALID_ARG, "engram_debug_gate_key_form: form %d not 0, 1 or 2", form);
  set_gate_key_form(form);
  return ENGRAM_OK;
}

engram_status engram_gate_forward_fp8(const void* mem, int64_t n_tok, int32_t d_mem, int32_t d_model,
                                      int32_t n_branch, const void* const* h, const void* const* wk,
                                      const void* const* wv, const void* const* gq,
                                      const void* const* gk, float eps, engram_dtype dtype,
                                      engram_key_norm key_norm, void* const* out, float* gate_out,
                                      void* const* value_out, hipStream_t stream) {
  const char* fn = "engram_gate_forward_fp8";
  if (enum_arg(dtype) != ENGRAM_BF16) return fail(ENGRAM_ERR_UNSUPPORTED, "%s: operands must be bf16", fn);
  if (d_mem % 128 != 0)
    return fail(ENGRAM_ERR_UNSUPPORTED, "%s: d_mem must be a multiple of 128 (got %d)", fn, d_mem);
  GateArgs a;
  const engram_status st = gate_args(fn, mem, n_tok, d_mem, d_model, n_branch, h, wk, wv, gq, gk, eps, ENGRAM_BF16,
                                     enum_arg(key_norm), out, gate_out, value_out, a);
  if (st != ENGRAM_OK || n_tok == 0) return st;
  const size_t bytes = gate_bf16_scratch_bytes(a, true);
  return with_scratch(fn, bytes, stream, [&](void* p) {
    a.part_dot = (float*)p;
    launch_gate_bf16(a, true, stream);
  });
}

engram_status engram_gate_prepare_fp8(int32_t d_mem, int32_t d_model, int32_t n_branch, const void* const* wk,
                                      const void* const* wv, const void* const* gq, const void* const* gk,
                                      engram_key_norm key_norm, uint8_t* const* wk_codes, float* const* wk_scales,
                                      uint8_t* const* wv_codes, float* const* wv_scales, hipStream_t stream) {
  const char* fn = "engram_gate_prepare_fp8";
  if (d_mem <= 0 || d_model <= 0 || d_mem % 128 != 0 || d_model % 32 != 0)
    return fail(ENGRAM_ERR_UNSUPPORTED, "%s: d_mem must be a positive multiple of 128 and d_model of 32 (got %d, %d)",
                fn, d_mem, d_model);
  if (n_branch <= 0 || n_branch > ENGRAM_MAX_BRANCHES)
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: n_branch %d not in [1, %d]", fn, n_branch, ENGRAM_MAX_BRANCHES);
  if (!valid_key_norm(enum_arg(key_norm)))
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: unknown key_norm %d", fn, enum_arg(key_norm));
  if (wk == nullptr || wv == nullptr || wk_codes == nullptr || wk_scales == nullptr || wv_codes == nullptr ||
      wv_scales == nullptr || (key_norm == ENGRAM_KEY_NORM_MEMORY && (gq == nullptr || gk == nullptr)))
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: null pointer array", fn);
  GateArgs a;
  memset(&a, 0, sizeof a);
  for (int m = 0; m < n_branch; ++m) {
    const bool gains_ok = key_norm == ENGRAM_KEY_NORM_PROJECTED ||
                          (gq[m] != nullptr && gk[m] != nullptr && aligned(gq[m], 16) && aligned(gk[m], 16));
    if (wk[m] == nullptr || wv[m] == nullptr || !aligned(wk[m], 16) || !aligned(wv[m], 16) || !gains_ok ||
        wk_codes[m] == nullptr || wv_codes[m] == nullptr || !aligned(wk_codes[m], 16) || !aligned(wv_codes[m], 16) ||
        wk_scales[m] == nullptr || wv_scales[m] == nullptr || !aligned(wk_scales[m], 4) || !aligned(wv_scales[m], 4))
      return fail(ENGRAM_ERR_INVALID_ARG, "%s: branch %d: null or misaligned weights, gains or outputs", fn, m);
    a.wk[m] = wk[m];
    a.wv[m] = wv[m];
    if (key_norm == ENGRAM_KEY_NORM_MEMORY) {
      a.gq[m] = gq[m];
      a.gk[m] = gk[m];
    }
  }
  a.d_mem = d_mem;
  a.d_model = d_model;
  a.n_branch = n_branch;
  a.key_norm = (int32_t)key_norm;
  launch_prepare_fp8(a, wk_codes, wk_scales, wv_codes, wv_scales, stream);
  return check_launch(fn);
}

engram_status engram_gate_prepare(int32_t d_mem, int32_t d_model, int32_t n_branch, const void* const* wk,
                                  const void* const* gq, const void* const* gk, void* const* wk_folded,
                                  hipStream_t stream) {
  const char* fn = "engram_gate_prepare";
  if (wk_folded == nullptr) return fail(ENGRAM_ERR_INVALID_ARG, "%s: null output array", fn);
  GateArgs a;
  // the shape and weight checks of the bf16 gate (h and out are not used: no tokens)
  const engram_status st = gate_args(fn, nullptr, 0, d_mem, d_model, n_branch, wk, wk, wk, gq, gk, 0.f, ENGRAM_BF16,
                                     ENGRAM_KEY_NORM_MEMORY, wk_folded, nullptr, nullptr, a);
  if (st != ENGRAM_OK) return st;
  for (int m = 0; m < n_branch; ++m)
    if (wk_folded[m] == nullptr || !aligned(wk_folded[m], 16))
      return fail(ENGRAM_ERR_INVALID_ARG, "%s: branch %d: null or misaligned output", fn, m);
  launch_gate_fold(a, (uint16_t* const*)wk_folded, stream);
  return check_launch(fn);
}

engram_status engram_gate_forward_prepared(const void* mem, int64_t n_tok, int32_t d_mem, int32_t d_model,
                                           int32_t n_branch, const void* const* h, const void* const* wk_folded,
                                           const void* const* wv, float eps, void* const* out, float* gate_out,
                                           void* const* value_out, hipStream_t stream) {
  const char* fn = "engram_gate_forward_prepared";
  GateArgs a;
  // the gains are folded into wk_folded: the gain arguments of the checks get the
  // weights (valid, aligned and never read)
  const engram_status st = gate_args(fn, mem, n_tok, d_mem, d_model, n_branch, h, wk_folded, wv, wk_folded,
                                     wk_folded, eps, ENGRAM_BF16, ENGRAM_KEY_NORM_MEMORY, out, gate_out, value_out,
                                     a);
  if (st != ENGRAM_OK || n_tok == 0) return st;
  const size_t bytes = gate_bf16_scratch_bytes(a, false, true);
  return with_scratch(fn, bytes, stream, [&](void* p) {
    a.part_dot = (float*)p;
    launch_gate_bf16(a, false, stream, true);
  });
}

engram_status engram_lookup_gate(const int32_t* raw, int32_t batch, int64_t ld, int64_t t_begin, int64_t t_count,
                                 const int32_t* map, int32_t vocab, const int32_t* orders, int32_t n_orders,
                                 int32_t heads, const uint64_t* mult, const uint32_t* rows, int32_t pad_id,
                                 const void* const* tables, int32_t w, int32_t d_model, int32_t n_branch,
                                 const void* const* h, const void* const* wk, const void* const* wv,
                                 const void* const* gq, const void* const* gk, float eps, engram_key_norm key_norm,
                                 void* const* out, float* gate_out, void* const* value_out, int32_t* ids_out,
                                 int32_t* err_count, hipStream_t stream) {
  const char* fn = "engram_lookup_gate";
  HashArgs hs;
  bool empty = false;
  engram_status st = hash_args(fn, raw, batch, ld, t_begin, t_count, map, vocab, orders, n_orders, heads, mult,
                               rows, pad_id, ids_out, nullptr, err_count, false, hs, &empty);
  if (st != ENGRAM_OK) return st;
  const int nt = n_orders * heads;
  int64_t rows64[ENGRAM_MAX_TABLES];
  for (int b = 0; b < nt; ++b) rows64[b] = rows[b];
  const int64_t n_tok = empty ? 0 : (int64_t)batch * t_count;
  // the lookup's table checks (no index or memory-vector array: stand-ins keep the
  // null checks quiet)
  static const int32_t no_idx = 0;
  alignas(16) static char no_out[16];
  st = check_gather(fn, &no_idx, n_tok, nt, tables, rows64, w, ENGRAM_BF16, no_out);
  if (st != ENGRAM_OK) return st;
  // (check_gather has made w a multiple of 8) a k-step's 64 values of a token then span
  // at most two tables
  if (w < 64) return fail(ENGRAM_ERR_UNSUPPORTED, "%s: table rows of %d values; needs at least 64", fn, w);
  if (ids_out != nullptr && !aligned(ids_out, 4)) return fail(ENGRAM_ERR_INVALID_ARG, "%s: misaligned ids_out", fn);
  GateArgs a;
  // the gate's checks; the memory vectors are never stored (table 0 stands in for them)
  st = gate_args(fn, tables[0], n_tok, nt * w, d_model, n_branch, h, wk, wv, gq, gk, eps, ENGRAM_BF16,
                 enum_arg(key_norm), out, gate_out, value_out, a);
  if (st != ENGRAM_OK || n_tok == 0) return st;
  GatherSrc g;
  memset(&g, 0, sizeof g);
  for (int b = 0; b < nt; ++b) {
    g.tab[b] = (const char*)tables[b];
    g.rows[b] = hs.rows[b];
    g.barrett[b] = hs.barrett[b];
    g.order[b] = hs.order[b];
    for (int j = 0; j < ENGRAM_MAX_ORDER; ++j) g.mult[b][j] = hs.mult[b][j];
  }
  g.n_tables = nt;
  g.cpr = w / 8;
  const size_t gate_bytes = gate_bf16_scratch_bytes(a, false);
  const size_t bytes = gate_bytes + (((size_t)n_tok * sizeof(int4) + 255) & ~(size_t)255);
  return with_scratch(fn, bytes, stream, [&](void* p) {
    a.part_dot = (float*)p;
    g.ids = (const int4*)((char*)p + gate_bytes);
    launch_gate_ids(hs, (int4*)g.ids, stream);
    launch_gate_bf16(a, false, stream, false, &g);
  });
}

engram_status engram_gate_forward_fp8q(const uint8_t* codes, const float* scales, const float* sumsq, int64_t n_tok,
                                       int32_t d_mem, int32_t d_model, int32_t n_branch, const void* const* h,
                                       const uint8_t* const* wk_codes, const float* const* wk_scales,
                                       const uint8_t* const* wv_codes, const float* const* wv_scales,
                                       const void* const* gq, const void* const* gk, float eps,
                                       engram_key_norm key_norm, void* const* out, float* gate_out,
                                       void* const* value_out, hipStream_t stream) {
  const char* fn = "engram_gate_forward_fp8q";
  if (d_mem % 128 != 0)
    return fail(ENGRAM_ERR_UNSUPPORTED, "%s: d_mem must be a multiple of 128 (got %d)", fn, d_mem);
  if (wk_scales == nullptr || wv_scales == nullptr) return fail(ENGRAM_ERR_INVALID_ARG, "%s: null scale array", fn);
  GateArgs a;
  const engram_status st = gate_args(fn, codes, n_tok, d_mem, d_model, n_branch, h, (const void* const*)wk_codes,
                                     (const void* const*)wv_codes, gq, gk, eps, ENGRAM_BF16, enum_arg(key_norm), out,
                                     gate_out, value_out, a);
  if (st != ENGRAM_OK) return st;
  for (int m = 0; m < n_branch; ++m) {
    if (wk_scales[m] == nullptr || wv_scales[m] == nullptr || !aligned(wk_scales[m], 4) || !aligned(wv_scales[m], 4))
      return fail(ENGRAM_ERR_INVALID_ARG, "%s: branch %d: null or misaligned weight scales", fn, m);
    a.sk[m] = wk_scales[m];
    a.sv[m] = wv_scales[m];
  }
  if (n_tok == 0) return ENGRAM_OK;
  if (scales == nullptr || !aligned(scales, 4) || (sumsq != nullptr && !aligned(sumsq, 4)) ||
      (key_norm == ENGRAM_KEY_NORM_MEMORY && sumsq == nullptr))
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: null or misaligned scales/sumsq (sumsq is needed for the "
                "memory-side key norm)", fn);
  a.se = scales;
  a.e_ssq = sumsq;
  const size_t bytes = gate_bf16_scratch_bytes(a, true, true);
  return with_scratch(fn, bytes, stream, [&](void* p) {
    a.part_dot = (float*)p;
    launch_gate_bf16(a, true, stream, true);
  });
}

engram_status engram_conv_forward(const void* value, int32_t batch, int64_t seq, int32_t d_model,
                                  const void* w, const void* gamma, int32_t taps, int32_t dilation,
                                  float eps, engram_dtype dtype, void* out, hipStream_t stream) {
  const char* fn = "engram_conv_forward";
  if (batch < 0 || seq < 0 || d_model <= 0)
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: bad sizes batch=%d seq=%lld d_model=%d", fn, batch,
                (long long)seq, d_model);
  if (!valid_dtype(enum_arg(dtype))) return fail(ENGRAM_ERR_INVALID_ARG, "%s: unknown dtype", fn);
  if (!(eps >= 0.f)) return fail(ENGRAM_ERR_INVALID_ARG, "%s: eps must be >= 0", fn);
  if (taps < 1 || taps > ENGRAM_CONV_MAX_TAPS)
    return fail(ENGRAM_ERR_UNSUPPORTED, "%s: taps %d not in [1, %d]", fn, taps, ENGRAM_CONV_MAX_TAPS);
  if (dilation < 1 || dilation > ENGRAM_CONV_MAX_DILATION)
    return fail(ENGRAM_ERR_UNSUPPORTED, "%s: dilation %d not in [1, %d]", fn, dilation,
                ENGRAM_CONV_MAX_DILATION);
  if (((int64_t)d_model * (int64_t)dtype_size(dtype)) % 16 != 0)
    return fail(ENGRAM_ERR_UNSUPPORTED, "%s: d_model * element size must be a multiple of 16 (d_model %d)",
                fn, d_model);
  if (w == nullptr || gamma == nullptr || !aligned(w, 16) || !aligned(gamma, 16))
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: null or misaligned w/gamma", fn);
  if (batch == 0 || seq == 0) return ENGRAM_OK;
  if (value == nullptr || out == nullptr || !aligned(value, 16) || !aligned(out, 16))
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: null or misaligned value/out", fn);
  const int64_t rows = (int64_t)batch * seq;
  const size_t row_bytes = (size_t)d_model * dtype_size(dtype);
  const char *v0 = (const char*)value, *o0 = (const char*)out;
  if (v0 < o0 + rows * row_bytes && o0 < v0 + rows * row_bytes)
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: out overlaps value", fn);
  if ((uint64_t)seq * row_bytes >= (1ull << 32))
    return fail(ENGRAM_ERR_UNSUPPORTED, "%s: one sequence's values exceed 4 GiB", fn);
  // workgroups of the apply kernel: 64-token blocks x 256-byte column slabs per sequence
  const int64_t slabs = ((int64_t)row_bytes / 16 + 15) / 16;
  if (rows / 4 + 1 >= (1ll << 31) || (int64_t)batch * ((seq + 63) / 64) * slabs >= (1ll << 31))
    return fail(ENGRAM_ERR_UNSUPPORTED, "%s: too many tokens for one launch", fn);
  ConvArgs a;
  memset(&a, 0, sizeof a);
  a.value = value;
  a.out = out;
  a.w = w;
  a.gamma = gamma;
  a.seq = seq;
  a.batch = batch;
  a.d_model = d_model;
  a.taps = taps;
  a.dil = dilation;
  a.eps = eps;
  const bool bf16 = enum_arg(dtype) == ENGRAM_BF16;
  return with_scratch(fn, conv_scratch_bytes(a, bf16), stream, [&](void* p) {
    a.inv = p;
    launch_conv(a, bf16, stream);
  });
}

engram_status engram_quantize_fp8(const void* src, int64_t rows, int32_t cols, engram_dtype dtype, uint8_t* codes,
                                  float* scales, float* sumsq, hipStream_t stream) {
  const char* fn = "engram_quantize_fp8";
  if (rows < 0 || cols <= 0) return fail(ENGRAM_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (!valid_dtype(enum_arg(dtype))) return fail(ENGRAM_ERR_INVALID_ARG, "%s: unknown dtype", fn);
  if (cols % 16 != 0) return fail(ENGRAM_ERR_UNSUPPORTED, "%s: cols %d not a multiple of 16", fn, cols);
  if (rows == 0) return ENGRAM_OK;
  if (src == nullptr || codes == nullptr || scales == nullptr || !aligned(src, 16) || !aligned(codes, 16) ||
      !aligned(scales, 4) || (sumsq != nullptr && !aligned(sumsq, 4)))
    return fail(ENGRAM_ERR_INVALID_ARG, "%s: null or misaligned pointer", fn);
  if ((rows + 3) / 4 >= (1ll << 31)) return fail(ENGRAM_ERR_UNSUPPORTED, "%s: too many rows", fn);
  launch_quant_rows(src, dtype == ENGRAM_BF16, rows, cols, nullptr, nullptr, codes, scales, sumsq, stream);
  return check_launch(fn);
}

engram_status engram_host_alloc(size_t bytes, void** ptr) {
  if (ptr == nullptr) return fail(ENGRAM_ERR_INVALID_ARG, "engram_host_alloc: null ptr");
  *ptr = nullptr;
  if (bytes == 0) return fail(ENGRAM_ERR_INVALID_ARG, "engram_host_alloc: zero bytes");
  const hipError_t e = hipHostMalloc(ptr, bytes, hipHostMallocMapped | hipHostMallocPortable);
  if (e != hipSuccess) {
    *ptr = nullptr;
    (void)hipGetLastError();  // not to be reported again by a later call's launch check
    return hip_fail(e, "engram_host_alloc: hipHostMalloc");
  }
  return ENGRAM_OK;
}

engram_status engram_host_free(void* ptr) {
  if (ptr == nullptr) return ENGRAM_OK;
  const hipError_t e = hipHostFree(ptr);
  if (e != hipSuccess) return hip_fail(e, "engram_host_free: hipHostFree");
  return ENGRAM_OK;
}

}  // extern "C"
