// row_ceiling.hip -- measurement probes for the benchmark, not part of the method's path:
// what the memory system delivers for the access pattern of the table gather, so that the
// gather's rate can be stated against a measured ceiling as well as the HBM spec peak.
//
//   engram_probe_row_reads: reads n random rows of row_bytes (given as row indices into
//     a [rows][row_bytes] table, 16-byte aligned rows) and writes nothing but one word
//     per thread (an XOR of what it read, so the loads cannot be dropped).  The layout is
//     the gather's: lanes take consecutive 16-byte chunks of the concatenation of a
//     thread row's rows (here one table, `rows_per_group` rows side by side), U groups
//     per thread in flight.  Works on device tables and on device mappings of pinned
//     host tables alike.
//   engram_probe_stream_reads: reads n_bytes contiguously the same way (the plain read
//     ceiling of the memory behind the pointer).
// Both are ordinary kernels on the caller's stream; the benchmark times them with events.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int U = 8;

__global__ __launch_bounds__(1024) void probe_rows_kernel(const char* __restrict__ table, const int32_t* __restrict__ idx,
                                                          int64_t n_groups, int cpr, int rows_per_group,
                                                          uint32_t* __restrict__ sink) {
  const int c = threadIdx.x;          // chunk of the group's concatenated rows
  const int j = c / cpr;              // which row of the group
  const int k = c - j * cpr;          // chunk inside the row
  const int64_t row_bytes = (int64_t)cpr * 16;
  const int64_t g0 = ((int64_t)blockIdx.x * U) * blockDim.y + threadIdx.y;
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t g = g0 + (int64_t)u * blockDim.y;
    v[u] = u32x4{0u, 0u, 0u, 0u};
    if (g < n_groups) {
      const int64_t r = idx[g * rows_per_group + j];
      v[u] = *reinterpret_cast<const u32x4*>(table + r * row_bytes + k * 16);
    }
  }
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  sink[(int64_t)blockIdx.x * blockDim.x * blockDim.y + threadIdx.y * blockDim.x + threadIdx.x] = x;
}

__global__ __launch_bounds__(256) void probe_stream_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                           uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t x = 0;
  for (int64_t i = t; i < n16; i += stride * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = i + u * stride < n16 ? src[i + u * stride] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  sink[t] = x;
}

}  // namespace

extern "C" {

// n_groups groups of rows_per_group rows (idx: [n_groups][rows_per_group] row numbers of
// one table, each < the table's rows); row_bytes % 16 == 0 and rows_per_group * row_bytes
// / 16 <= 1024.  sink: device uint32 [probe_rows_sink_words(...)].  Returns 0, or -1 for
// bad arguments (nothing launched).
int64_t engram_probe_rows_sink_words(int64_t n_groups, int32_t row_bytes, int32_t rows_per_group) {
  const int cpt = rows_per_group * (row_bytes / 16);
  int ty = 256 / cpt;
  if (ty < 1) ty = 1;
  const int64_t blocks = (n_groups + (int64_t)ty * U - 1) / ((int64_t)ty * U);
  return blocks * cpt * ty;
}

int engram_probe_row_reads(const void* table, int32_t row_bytes, const int32_t* idx, int64_t n_groups,
                           int32_t rows_per_group, uint32_t* sink, hipStream_t stream) {
  if (table == nullptr || idx == nullptr || sink == nullptr || row_bytes <= 0 || row_bytes % 16 != 0 ||
      rows_per_group <= 0 || n_groups <= 0 || (int64_t)rows_per_group * (row_bytes / 16) > 1024)
    return -1;
  const int cpr = row_bytes / 16;
  const int cpt = rows_per_group * cpr;
  int ty = 256 / cpt;
  if (ty < 1) ty = 1;
  const int64_t blocks = (n_groups + (int64_t)ty * U - 1) / ((int64_t)ty * U);
  hipLaunchKernelGGL(probe_rows_kernel, dim3((unsigned)blocks), dim3(cpt, ty), 0, stream, (const char*)table, idx,
                     n_groups, cpr, rows_per_group, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// sink: device uint32 [blocks * 256] with blocks = 8192.
int engram_probe_stream_reads(const void* src, int64_t n_bytes, uint32_t* sink, hipStream_t stream) {
  if (src == nullptr || sink == nullptr || n_bytes <= 0 || n_bytes % 16 != 0) return -1;
  hipLaunchKernelGGL(probe_stream_kernel, dim3(8192), dim3(256), 0, stream, (const u32x4*)src, n_bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
