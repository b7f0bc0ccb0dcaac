// gather.hip -- table row lookup and concatenation into the memory vector.
// "Conditional Memory via Scalable Lookup", section 2.2, Eq. (1)-(2): each
// (token, table) index selects one row of that table, and the rows of all
// tables are concatenated (order-major, head-minor) into e_t.
//
// Layout of the work: the output row of one token is n_tables * row_bytes
// bytes, cut into 16-byte chunks.  threadIdx.x is the chunk number inside that
// row, so (a) a wavefront stores consecutive 16-byte chunks of the output
// (fully coalesced 1-KB stores), (b) the row_bytes/16 lanes that read one table
// row read it as one contiguous span, and (c) each lane's table number and
// offset inside the row are fixed for the whole kernel.  threadIdx.y picks the
// token inside the workgroup, and each thread walks U tokens with all U loads
// issued before the stores, to keep enough 16-byte requests in flight to cover
// HBM latency (and, for host-resident tables, PCIe latency).
//
// The same kernel serves engram_prefetch_host: there the table pointers are
// device mappings of pinned host memory and every load crosses PCIe.
#include "engram_internal.h"

namespace engram {
namespace {

template <int U>
__global__ __launch_bounds__(1024) void gather_kernel(const GatherArgs a) {
  const int c = threadIdx.x;
  const int cpr = a.chunks_per_row;
  const int b = c / cpr;
  const int k = c - b * cpr;
  const char* tab = a.table[b];
  const int64_t rows = a.rows[b];
  const int64_t row_bytes = (int64_t)cpr * 16;
  const int64_t out_row_bytes = row_bytes * a.n_tables;
  const int64_t t_first = ((int64_t)blockIdx.x * U) * blockDim.y + threadIdx.y;
  const int nt = a.n_tables;

  uint4 v[U];
  int bad = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t t = t_first + (int64_t)u * blockDim.y;
    v[u] = make_uint4(0u, 0u, 0u, 0u);
    if (t < a.n_tok) {
      const int64_t r = a.idx[t * nt + b];
      if ((uint64_t)r < (uint64_t)rows) {
        v[u] = *reinterpret_cast<const uint4*>(tab + r * row_bytes + k * 16);
      } else {
        bad += (k == 0);  // one count per bad (token, table) pair
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t t = t_first + (int64_t)u * blockDim.y;
    if (t < a.n_tok) *reinterpret_cast<uint4*>(a.out + t * out_row_bytes + c * 16) = v[u];
  }
  if (bad != 0 && a.err_count != nullptr) atomicAdd(a.err_count, bad);
}

}  // namespace

void launch_gather(const GatherArgs& a, bool host_source, hipStream_t s) {
  const int cpt = a.n_tables * a.chunks_per_row;  // <= 1024, checked by the caller
  if (host_source) {
    // one token per thread: every 16-byte PCIe read of the step is issued at once
    int ty = 512 / cpt;
    if (ty < 1) ty = 1;
    const int64_t blocks = (a.n_tok + ty - 1) / ty;
    hipLaunchKernelGGL(gather_kernel<1>, dim3((unsigned)blocks), dim3(cpt, ty), 0, s, a);
  } else {
    // eight tokens per thread, about 256 threads per workgroup: measured the fastest of
    // U in {2, 4, 8} x {256, 512, 1024} threads at 16 tables of 160-byte rows (all
    // within 5 %; the random rows, not the launch shape, set the pace)
    constexpr int U = 8;
    int ty = 256 / cpt;
    if (ty < 1) ty = 1;
    const dim3 block(cpt, ty);
    const int64_t blocks = (a.n_tok + (int64_t)ty * U - 1) / ((int64_t)ty * U);
    hipLaunchKernelGGL(gather_kernel<U>, dim3((unsigned)blocks), block, 0, s, a);
  }
}

}  // namespace engram
