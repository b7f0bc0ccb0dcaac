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
//                      16-byte chunks).  It stages the slab's V~ rows of the block and
//                      the (TAPS-1)*dil rows of causal history before it in LDS, already
//                      normalized (V~ * inv, in fp32; rows before the sequence start are
//                      zero, so every tap reads the tile without a branch), six rows per
//                      thread in flight, with the thread's output chunks loaded alongside.
//                      Each thread then takes one chunk column and TB / RPP tokens RPP
//                      rows apart; its kernel weights (CH channels x TAPS taps, contiguous,
//                      with gamma folded in) sit in registers, so a tap is one FMA per
//                      element.  Global memory sees each V~ element once (plus the history
//                      rows shared with the previous block).
// Workgroups are numbered so that each XCD runs a contiguous range of (token block,
// slab) pairs in order: the history rows a block needs were read by the block of the
// same slab just before it on the same XCD and are still in that XCD's L2.
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int NTHR_C = 256;
constexpr int SW = 16;              // 16-byte chunks per slab
constexpr int RPP = NTHR_C / SW;    // token rows per pass
constexpr int TB = 64;              // tokens per workgroup
constexpr int HALO_MAX = (ENGRAM_CONV_MAX_TAPS - 1) * ENGRAM_CONV_MAX_DILATION;
constexpr int N_XCD = 8;
// the normalized tile at the largest history fits one workgroup's LDS (8 fp32 values per
// bf16 chunk, or 4 fp64 values per fp32 chunk: 32 bytes per chunk either way)
static_assert((TB + HALO_MAX) * SW * 32 <= 160 * 1024, "conv tile exceeds LDS");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// SiLU(z) = z / (1 + e^-z) from the hardware exp2 and reciprocal (each about 1 ulp in
// fp32).  The IEEE expf and division cost ~40 instructions per element, which made the
// kernel ALU-bound; this form is four.  Limits: z -> -inf gives e^-z = inf, 1/inf = 0 and
// -0; z -> +inf gives z.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(z * -1.44269504088896341f));
}
// fp64 form, for fp32 storage (an output that nearly cancels, base + SiLU(z) ~ 0, would
// expose the fp32 form's errors as a large relative error; fp32 values are tiny workloads)
__device__ __forceinline__ double silu(double z) { return z / (1.0 + exp(-z)); }

// The arithmetic type per storage type: fp32 for bf16 (values are rounded to bf16
// anyway), fp64 for fp32 (the output is rounded to fp32 once).
template <typename T> struct Acc;
template <> struct Acc<uint16_t> {
  using type = float;
  using vec4 = float4;
  __device__ static vec4 make(type a, type b, type c, type d) { return make_float4(a, b, c, d); }
};
template <> struct Acc<float> {
  using type = double;
  using vec4 = double4;
  __device__ static vec4 make(type a, type b, type c, type d) { return make_double4(a, b, c, d); }
};

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
    for (int i = 0; i < 4; ++i)  // round to nearest even, two per v_cvt_pk_bf16_f32
      v[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x[2 * i], x[2 * i + 1]}, bf16x2));
    *reinterpret_cast<u32x4*>(p) = v;
  }
};

// inv[r] = 1 / sqrt(mean(V~[r]^2) + eps) for every row r of the batch, a wavefront per row
// (in the arithmetic type A: a.inv holds A values).
template <typename T>
__global__ __launch_bounds__(NTHR_C) void conv_rms_kernel(const ConvArgs a) {
  using A = typename Acc<T>::type;
  constexpr int CH = Chunk<T>::CH;
  const int64_t n_rows = (int64_t)a.batch * a.seq;
  const int64_t r = (int64_t)blockIdx.x * (NTHR_C / 64) + (threadIdx.x >> 6);
  if (r >= n_rows) return;  // uniform per wavefront
  const int lane = threadIdx.x & 63;
  const int chunks = a.d_model / CH;
  const T* row = reinterpret_cast<const T*>(a.value) + r * a.d_model;
  A ss = 0;
  for (int c0 = lane; c0 < chunks; c0 += 8 * 64) {  // up to eight chunks per lane in flight
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = c0 + u * 64;
      v[u] = c < chunks ? *reinterpret_cast<const u32x4*>(row + c * CH) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float x[CH];
      Chunk<T>::load(&v[u], x);
#pragma unroll
      for (int i = 0; i < CH; ++i) ss += (A)x[i] * (A)x[i];
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if (lane == 0) reinterpret_cast<A*>(a.inv)[r] = (A)1 / sqrt(ss / (A)a.d_model + (A)a.eps);
}

template <typename T, int TAPS>
__global__ __launch_bounds__(NTHR_C) void conv_apply_kernel(const ConvArgs a, int nblk_t, int n_slab) {
  using A = typename Acc<T>::type;
  using A4 = typename Acc<T>::vec4;
  constexpr int CH = Chunk<T>::CH;
  constexpr int H = CH / 4;     // 4-element pieces per chunk
  constexpr int KT = TB / RPP;  // tokens per thread
  // [TB + halo][H][SW] vectors of four A: the normalized rows V~ * inv of the slab (gamma
  // is folded into the weights), zero before the sequence start
  extern __shared__ __attribute__((aligned(32))) char s_raw[];
  A4* s_tile = reinterpret_cast<A4*>(s_raw);
  // XCD-contiguous numbering: hardware block id b goes to XCD b % N_XCD
  const int nb = gridDim.x, q = nb / N_XCD, rem = nb % N_XCD;
  const int xcd = blockIdx.x % N_XCD;
  const int L = xcd * q + (xcd < rem ? xcd : rem) + blockIdx.x / N_XCD;
  const int slab = L % n_slab;
  const int tb = (L / n_slab) % nblk_t;
  const int b = L / (n_slab * nblk_t);

  const int halo = (TAPS - 1) * a.dil;
  const int nrows = TB + halo;
  const int seq = (int)a.seq;      // positions and byte offsets within one sequence fit
  const int t0 = tb * TB;          // 32 bits (the caller limits a sequence to 4 GiB)
  const int first = t0 - halo;     // tile row i holds position first + i
  const int64_t row0 = (int64_t)b * a.seq;
  const int chunks = a.d_model / CH;
  const int cl = (int)(threadIdx.x % SW), rr = (int)(threadIdx.x / SW);
  const int c = slab * SW + cl;
  const bool col_ok = c < chunks;
  const int c0 = col_ok ? c * CH : 0;
  const char* V = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.value) + row0 * a.d_model + c0);
  char* O = reinterpret_cast<char*>(reinterpret_cast<T*>(a.out) + row0 * a.d_model + c0);
  const A* inv = reinterpret_cast<const A*>(a.inv) + row0;
  const uint32_t ld = (uint32_t)a.d_model * (uint32_t)sizeof(T);

  // this thread's output chunks (tokens t0 + rr + RPP k), loaded first: they are
  // independent of the staging and the barrier
  u32x4 ov[KT];
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    const int t = t0 + rr + RPP * k;
    ov[k] = (col_ok && t < seq) ? *reinterpret_cast<const u32x4*>(O + (uint32_t)t * ld) : u32x4{0, 0, 0, 0};
  }
  // stage the tile, SR rows per thread in flight at once, normalized on the way in
  constexpr int SR = 6;
  for (int i0 = 0; i0 < nrows; i0 += SR * RPP) {
    u32x4 v[SR];
    A sc[SR];
#pragma unroll
    for (int u = 0; u < SR; ++u) {
      const int i = i0 + u * RPP + rr;
      const int ts = first + i;
      const bool ok = i < nrows && ts >= 0 && ts < seq;
      v[u] = (ok && col_ok) ? *reinterpret_cast<const u32x4*>(V + (uint32_t)ts * ld) : u32x4{0, 0, 0, 0};
      sc[u] = ok ? inv[ts] : (A)0;
    }
#pragma unroll
    for (int u = 0; u < SR; ++u) {
      const int i = i0 + u * RPP + rr;
      if (i < nrows) {
        float x[CH];
        Chunk<T>::load(&v[u], x);
#pragma unroll
        for (int hh = 0; hh < H; ++hh)
          s_tile[(i * H + hh) * SW + cl] = Acc<T>::make((A)x[4 * hh] * sc[u], (A)x[4 * hh + 1] * sc[u],
                                                         (A)x[4 * hh + 2] * sc[u], (A)x[4 * hh + 3] * sc[u]);
      }
    }
  }
  float g[CH], wl[CH * TAPS];  // the chunk's gains and kernel weights as stored
  A wg[CH * TAPS];             // wg[i * TAPS + j] = w[c0 + i][j] * gamma[c0 + i]
  Chunk<T>::load(reinterpret_cast<const T*>(a.gamma) + c0, g);
#pragma unroll
  for (int k = 0; k < TAPS; ++k)
    Chunk<T>::load(reinterpret_cast<const T*>(a.w) + (int64_t)c0 * TAPS + k * CH, wl + k * CH);
#pragma unroll
  for (int i = 0; i < CH; ++i)
#pragma unroll
    for (int j = 0; j < TAPS; ++j) wg[i * TAPS + j] = (A)wl[i * TAPS + j] * (A)g[i];
  __syncthreads();
  if (!col_ok) return;  // no barrier follows

#pragma unroll
  for (int k = 0; k < KT; ++k) {
    const int tl = rr + RPP * k;  // position t0 + tl, tile row tl + halo
    if (t0 + tl >= seq) break;
    A z[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) z[i] = 0;
#pragma unroll
    for (int j = 0; j < TAPS; ++j) {
      const int row = tl + halo - j * a.dil;  // >= 0; rows before the sequence start are zero
#pragma unroll
      for (int hh = 0; hh < H; ++hh) {
        const A4 n = s_tile[(row * H + hh) * SW + cl];
        z[4 * hh] = fma(wg[(4 * hh) * TAPS + j], n.x, z[4 * hh]);
        z[4 * hh + 1] = fma(wg[(4 * hh + 1) * TAPS + j], n.y, z[4 * hh + 1]);
        z[4 * hh + 2] = fma(wg[(4 * hh + 2) * TAPS + j], n.z, z[4 * hh + 2]);
        z[4 * hh + 3] = fma(wg[(4 * hh + 3) * TAPS + j], n.w, z[4 * hh + 3]);
      }
    }
    float o[CH];
    Chunk<T>::load(&ov[k], o);
#pragma unroll
    for (int i = 0; i < CH; ++i) o[i] = (float)((A)o[i] + silu(z[i]));
    Chunk<T>::store(O + (uint32_t)(t0 + tl) * ld, o);
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
  const size_t tile_bytes =
      (size_t)(TB + (a.taps - 1) * a.dil) * SW * Chunk<T>::CH * sizeof(typename Acc<T>::type);
  switch (a.taps) {
#define ENGRAM_CONV_CASE(K) \
  case K: hipLaunchKernelGGL((conv_apply_kernel<T, K>), grid, dim3(NTHR_C), tile_bytes, s, a, nblk_t, n_slab); break;
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

size_t conv_scratch_bytes(const ConvArgs& a, bool bf16) {
  return (size_t)a.batch * (size_t)a.seq * (bf16 ? sizeof(float) : sizeof(double));
}

}  // namespace engram
