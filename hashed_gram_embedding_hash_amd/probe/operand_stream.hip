// operand_stream.hip -- measurement probes for the benchmark, not part of the method's path:
// how fast a workgroup moves L2-resident operand bytes into LDS by the two routes a matrix
// kernel's main loop can take, with one workgroup of 256 threads per CU (96 KB of LDS each).
//
//   engram_probe_lds_dma:  every iteration each wave issues 16 direct global->LDS loads of
//     16 bytes per lane (global_load_lds_dwordx4: 1 KB per instruction, 64 KB per workgroup),
//     waits for them and meets the others at a barrier -- the gate's k-step without the
//     matrix work;
//   engram_probe_lds_vgpr: the same 64 KB per iteration as 16 ordinary 16-byte loads per
//     lane into registers, then 16 ds_write_b128 stores into LDS and a barrier.
// The source is a small buffer (the caller passes 2 MB) that every workgroup of an XCD reads,
// so after the first pass the loads hit the L2.  Each workgroup finally writes one word per
// thread of what it stored in LDS (so that nothing can be dropped).  Both are ordinary
// kernels on the caller's stream; the benchmark times them with events.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;
constexpr int LDS_BYTES = 96 * 1024;  // more than half the CU's LDS: one workgroup per CU
constexpr int CHUNKS = 4096;          // 16-byte chunks per workgroup and iteration (64 KB)

// One 16-byte-per-lane direct load: lane l's 16 bytes from src land at LDS byte address
// lds + 16 l (lds wave-uniform, through M0; one wait state between writing M0 and the load).
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

__device__ __forceinline__ int64_t chunk_of(int64_t it, int wave, int i, int lane, int64_t n_chunks) {
  return ((int64_t)blockIdx.x * CHUNKS + it * CHUNKS + (int64_t)((wave * 16 + i) * 64 + lane)) % n_chunks;
}

__global__ __launch_bounds__(256) void probe_lds_dma_kernel(const u32x4* __restrict__ src, int64_t n_chunks,
                                                            int iters, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr)smem;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) dma16(src + chunk_of(it, wave, i, lane, n_chunks), lds0 + (wave * 16 + i) * 1024);
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0): this wave's loads have landed
    __syncthreads();
  }
  sink[(int64_t)blockIdx.x * 256 + tid] = reinterpret_cast<const uint32_t*>(smem)[tid * 4];
}

__global__ __launch_bounds__(256) void probe_lds_vgpr_kernel(const u32x4* __restrict__ src, int64_t n_chunks,
                                                             int iters, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int it = 0; it < iters; ++it) {
    u32x4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = src[chunk_of(it, wave, i, lane, n_chunks)];
#pragma unroll
    for (int i = 0; i < 16; ++i) *reinterpret_cast<u32x4*>(smem + (wave * 16 + i) * 1024 + lane * 16) = v[i];
    __syncthreads();
  }
  sink[(int64_t)blockIdx.x * 256 + tid] = reinterpret_cast<const uint32_t*>(smem)[tid * 4];
}

}  // namespace

extern "C" {

// src: device, n_bytes (a multiple of 16, at least 64 KB); sink: device uint32 [blocks * 256].
// Returns 0, or -1 for bad arguments (nothing launched).
int engram_probe_lds_dma(const void* src, int64_t n_bytes, int32_t blocks, int32_t iters, uint32_t* sink,
                         hipStream_t stream) {
  if (src == nullptr || sink == nullptr || n_bytes < 65536 || n_bytes % 16 != 0 || blocks <= 0 || iters <= 0)
    return -1;
  hipLaunchKernelGGL(probe_lds_dma_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const u32x4*)src,
                     n_bytes / 16, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int engram_probe_lds_vgpr(const void* src, int64_t n_bytes, int32_t blocks, int32_t iters, uint32_t* sink,
                          hipStream_t stream) {
  if (src == nullptr || sink == nullptr || n_bytes < 65536 || n_bytes % 16 != 0 || blocks <= 0 || iters <= 0)
    return -1;
  hipLaunchKernelGGL(probe_lds_vgpr_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const u32x4*)src,
                     n_bytes / 16, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
