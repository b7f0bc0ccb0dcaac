// conv.hip -- short depthwise causal convolution over the gated values.
// "Conditional Memory via Scalable Lookup", section 2.3, Eq. (5): with V~ the gated
// values alpha_t v_t of one sequence, the module's output is
//   Y = SiLU(Conv1D(RMSNorm(V~))) + V~,
// a depthwise convolution over time, causal within each sequence.  The gate already
// adds V~ to the residual, so these kernels add the remaining term in place:
//   out[t, c] += SiLU( sum_j w[c][j] * n[t - j*dil, c] ),
//   n[t] = V~[t] * inv[t] * gamma,   inv[t] = 1 / sqrt(mean_c V~[t, c]^2 + eps).
//
// Two launches, both bound by HBM bandwidth:
//   conv_rms_kernel    a wavefront per token row reduces sum(V~^2) and writes inv[t]
//                      (4 bytes per token into the library scratch);
//   conv_apply_kernel  a workgroup per (sequence, block of TB tokens, slab of SW
//                      16-byte chunks).  Its threads take one chunk column each and
//                      walk the block's tokens RPP rows apart, so every wavefront
//                      reads and writes 512 contiguous bytes of two rows.  The kernel
//                      weights of a chunk (CH channels x TAPS taps, contiguous) and
//                      its gains stay in registers for the whole block; the block's
//                      inv values, with the (TAPS-1)*dil rows of causal history
//                      before it, are staged in LDS.  The taps j > 0 re-read rows
//                      that tap 0 of a nearby row read a few passes earlier, so they
//                      are served by the caches.
// Workgroups are numbered so that each XCD runs a contiguous range of (token block,
// slab) pairs in order: the history rows a block needs were read by the block of the
// same slab just before it on the same XCD and are still in that XCD's L2.
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int NTHR_C = 256;
constexpr int SW = 32;              // 16-byte chunks per slab
constexpr int RPP = NTHR_C / SW;    // token rows per pass
constexpr int TB = 64;              // tokens per workgroup
constexpr int HALO_MAX = (ENGRAM_CONV_MAX_TAPS - 1) * ENGRAM_CONV_MAX_DILATION;
constexpr int N_XCD = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float silu(float z) { return z / (1.f + expf(-z)); }

// One 16-byte chunk: CH elements of the storage type, converted to/from fp32.
template <typename T> struct Chunk;
template <> struct Chunk<float> {
  static constexpr int CH = 4;
  __device__ static void load(const void* p, float* x) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(v[i]);
  }
  __device__ static void store(void* p, const float* x) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(x[i]);
    *reinterpret_cast<u32x4*>(p) = v;
  }
};
template <> struct Chunk<uint16_t> {  // bfloat16 bit patterns
  static constexpr int CH = 8;
  __device__ static void load(const void* p, float* x) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(v[i] << 16);
      x[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  __device__ static void store(void* p, const float* x) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 lo = (__bf16)x[2 * i], hi = (__bf16)x[2 * i + 1];  // round to nearest even
      v[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
             ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    *reinterpret_cast<u32x4*>(p) = v;
  }
};

// inv[r] = 1 / sqrt(mean(V~[r]^2) + eps) for every row r of the batch, a wavefront per row.
template <typename T>
__global__ __launch_bounds__(NTHR_C) void conv_rms_kernel(const ConvArgs a) {
  constexpr int CH = Chunk<T>::CH;
  const int64_t n_rows = (int64_t)a.batch * a.seq;
  const int64_t r = (int64_t)blockIdx.x * (NTHR_C / 64) + (threadIdx.x >> 6);
  if (r >= n_rows) return;  // uniform per wavefront
  const int lane = threadIdx.x & 63;
  const int chunks = a.d_model / CH;
  const T* row = reinterpret_cast<const T*>(a.value) + r * a.d_model;
  float ss = 0.f;
#pragma unroll 4
  for (int c = lane; c < chunks; c += 64) {
    float x[CH];
    Chunk<T>::load(row + c * CH, x);
#pragma unroll
    for (int i = 0; i < CH; ++i) ss += x[i] * x[i];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if (lane == 0) a.inv[r] = 1.f / sqrtf(ss / (float)a.d_model + a.eps);
}

template <typename T, int TAPS>
__global__ __launch_bounds__(NTHR_C) void conv_apply_kernel(const ConvArgs a, int nblk_t, int n_slab) {
  constexpr int CH = Chunk<T>::CH;
  __shared__ float s_inv[TB + HALO_MAX];
  // XCD-contiguous numbering: hardware block id b goes to XCD b % N_XCD
  const int nb = gridDim.x, q = nb / N_XCD, rem = nb % N_XCD;
  const int xcd = blockIdx.x % N_XCD;
  const int L = xcd * q + (xcd < rem ? xcd : rem) + blockIdx.x / N_XCD;
  const int slab = L % n_slab;
  const int tb = (L / n_slab) % nblk_t;
  const int b = L / (n_slab * nblk_t);

  const int halo = (TAPS - 1) * a.dil;
  const int64_t t0 = (int64_t)tb * TB;
  const int64_t first = t0 - halo;  // s_inv[i] belongs to position first + i
  const int64_t row0 = (int64_t)b * a.seq;
  for (int i = threadIdx.x; i < TB + halo; i += NTHR_C) {
    const int64_t ts = first + i;
    s_inv[i] = (ts >= 0 && ts < a.seq) ? a.inv[row0 + ts] : 0.f;
  }
  __syncthreads();

  const int chunks = a.d_model / CH;
  const int c = slab * SW + (int)(threadIdx.x % SW);
  if (c >= chunks) return;  // no barrier follows
  const int c0 = c * CH;
  const T* V = reinterpret_cast<const T*>(a.value) + row0 * a.d_model + c0;
  T* O = reinterpret_cast<T*>(a.out) + row0 * a.d_model + c0;

  float g[CH], w[CH * TAPS];  // w[i * TAPS + j]: channel c0 + i, tap j
  Chunk<T>::load(reinterpret_cast<const T*>(a.gamma) + c0, g);
#pragma unroll
  for (int k = 0; k < TAPS; ++k)
    Chunk<T>::load(reinterpret_cast<const T*>(a.w) + (int64_t)c0 * TAPS + k * CH, w + k * CH);

  const int64_t t_end = (t0 + TB < a.seq) ? t0 + TB : a.seq;
  for (int64_t t = t0 + (int)(threadIdx.x / SW); t < t_end; t += RPP) {
    float z[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) z[i] = 0.f;
#pragma unroll
    for (int j = 0; j < TAPS; ++j) {
      const int64_t ts = t - (int64_t)j * a.dil;
      if (ts >= 0) {
        float x[CH];
        Chunk<T>::load(V + ts * a.d_model, x);
        const float sc = s_inv[ts - first];
#pragma unroll
        for (int i = 0; i < CH; ++i) z[i] += w[i * TAPS + j] * (x[i] * sc * g[i]);
      }
    }
    float o[CH];
    Chunk<T>::load(O + t * a.d_model, o);
#pragma unroll
    for (int i = 0; i < CH; ++i) o[i] += silu(z[i]);
    Chunk<T>::store(O + t * a.d_model, o);
  }
}

template <typename T>
void launch_conv_t(const ConvArgs& a, hipStream_t s) {
  const int64_t n_rows = (int64_t)a.batch * a.seq;
  hipLaunchKernelGGL(conv_rms_kernel<T>, dim3((unsigned)((n_rows + 3) / 4)), dim3(NTHR_C), 0, s, a);
  const int nblk_t = (int)((a.seq + TB - 1) / TB);
  const int chunks = a.d_model / Chunk<T>::CH;
  const int n_slab = (chunks + SW - 1) / SW;
  const dim3 grid((unsigned)((int64_t)a.batch * nblk_t * n_slab));
  switch (a.taps) {
#define ENGRAM_CONV_CASE(K) \
  case K: hipLaunchKernelGGL((conv_apply_kernel<T, K>), grid, dim3(NTHR_C), 0, s, a, nblk_t, n_slab); break;
    ENGRAM_CONV_CASE(1) ENGRAM_CONV_CASE(2) ENGRAM_CONV_CASE(3) ENGRAM_CONV_CASE(4)
    ENGRAM_CONV_CASE(5) ENGRAM_CONV_CASE(6) ENGRAM_CONV_CASE(7) ENGRAM_CONV_CASE(8)
#undef ENGRAM_CONV_CASE
    default: break;  // the caller validated 1 <= taps <= ENGRAM_CONV_MAX_TAPS
  }
}

static_assert(ENGRAM_CONV_MAX_TAPS == 8, "one conv_apply_kernel instance per tap count");

}  // namespace

void launch_conv(const ConvArgs& a, bool bf16, hipStream_t s) {
  if (bf16)
    launch_conv_t<uint16_t>(a, s);
  else
    launch_conv_t<float>(a, s);
}

size_t conv_scratch_bytes(const ConvArgs& a) { return (size_t)a.batch * (size_t)a.seq * sizeof(float); }

}  // namespace engram
