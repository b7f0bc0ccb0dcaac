// compress.hip -- tokenizer compression lookup x' = P(x).
// "Conditional Memory via Scalable Lookup", section 2.2 (tokenizer compression):
// the surjection P from raw ids to canonical ids is precomputed, so at run time
// it is a table lookup.  The 4-byte-per-id map stays in L2 (517 KB for the
// 129,280-id vocabulary); the kernel is a streaming int32 read/write.
#include "engram_internal.h"

namespace engram {
namespace {

__global__ __launch_bounds__(256) void compress_kernel(const int32_t* raw, int64_t n,
                                                       const int32_t* __restrict__ map,
                                                       int32_t vocab, int32_t* out,
                                                       int32_t* err_count) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int32_t x = raw[i];
    const bool ok = (uint32_t)x < (uint32_t)vocab;
    out[i] = ok ? map[x] : -1;
    bad += ok ? 0 : 1;
  }
  if (err_count != nullptr) {
    // one atomic per wavefront that saw a bad id
    for (int off = 32; off > 0; off >>= 1) bad += __shfl_xor(bad, off, 64);
    if ((threadIdx.x & 63) == 0 && bad != 0) atomicAdd(err_count, bad);
  }
}

}  // namespace

void launch_compress(const int32_t* raw, int64_t n, const int32_t* map, int32_t vocab, int32_t* out,
                     int32_t* err_count, hipStream_t s) {
  const int threads = 256;
  int64_t blocks = (n + threads - 1) / threads;
  if (blocks > 8192) blocks = 8192;  // grid-stride beyond 2M ids
  hipLaunchKernelGGL(compress_kernel, dim3((unsigned)blocks), dim3(threads), 0, s, raw, n, map,
                     vocab, out, err_count);
}

}  // namespace engram
