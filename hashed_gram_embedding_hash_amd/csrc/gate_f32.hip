// gate_f32.hip -- context-aware gating for fp32 operands.
//
// Same definition as the bf16 path ("Conditional Memory via Scalable Lookup",
// section 2.3, Eq. (3)-(4), gated value, residual; section 2.4 Eq. (6) per
// branch), for fp32 tables, weights and hidden states.  fp32 inputs have no
// matrix-core path worth taking at the sizes this dtype is used for (tiny,
// launch-bound configurations), so one workgroup handles one (token, branch):
//   1. block reductions give sum(e^2) and sum(h^2);
//   2. RMSNorm(e) * gk is staged in LDS;
//   3. each wavefront takes output features in turn, its lanes read one row of
//      W_K (coalesced) against the staged vector and reduce across the wave;
//      q_i * k_i accumulates into the logit (with the projected key norm, the raw
//      k = W_K e goes to LDS first and its RMSNorm is applied to the reduced sums);
//   4. alpha = sigmoid(logit / sqrt(d_model)), then the same row-per-wavefront
//      loop over W_V writes out_i = h_i + alpha * v_i (and the gated value
//      alpha * v_i when it is asked for).
// The fp32 inputs are exact in fp64, and every product, sum, norm and the sigmoid are
// computed in fp64; each output is rounded to fp32 once.  fp32 sums over d_mem terms
// would carry errors of several units in the last place of their largest terms, which
// an output that nearly cancels (h + alpha v ~ 0, or v ~ 0 in the gated value) turns
// into a large relative error; this path costs nothing measurable either way.
// All reductions run in a fixed order, so results are bit-reproducible.
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int NTHR = 256;
constexpr int NWAVE = NTHR / 64;

__device__ __forceinline__ double wave_sum(double v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sum over the workgroup; every thread gets the result.
__device__ __forceinline__ double block_sum(double v, double* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < NWAVE; ++w) s += red[w];
  __syncthreads();
  return s;
}

__global__ __launch_bounds__(NTHR) void gate_f32_kernel(const GateArgs a) {
  extern __shared__ double s_en[];  // [d_mem] (+ [d_model] with the projected key norm)
  __shared__ double red[NWAVE];
  __shared__ double s_dot[NWAVE];

  const int64_t t = blockIdx.x;
  const int m = blockIdx.y;
  const int d_mem = a.d_mem, d_model = a.d_model;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* e = (const float*)a.mem + t * d_mem;
  const float* h = (const float*)a.h[m] + t * d_model;
  const float* wk = (const float*)a.wk[m];
  const float* wv = (const float*)a.wv[m];
  const float* gq = (const float*)a.gq[m];
  const float* gk = (const float*)a.gk[m];
  float* out = (float*)a.out[m] + t * d_model;
  float* vout = a.vout[m] != nullptr ? (float*)a.vout[m] + t * d_model : nullptr;
  const double eps = a.eps;

  double ss = 0.0;
  for (int j = threadIdx.x; j < d_mem; j += NTHR) ss += (double)e[j] * e[j];
  const double rms_e = sqrt(block_sum(ss, red) / d_mem + eps);
  double sh = 0.0;
  for (int i = threadIdx.x; i < d_model; i += NTHR) sh += (double)h[i] * h[i];
  const double rms_h = sqrt(block_sum(sh, red) / d_model + eps);

  double logit = 0.0;
  if (a.key_norm == ENGRAM_KEY_NORM_MEMORY) {
    for (int j = threadIdx.x; j < d_mem; j += NTHR) s_en[j] = (double)e[j] / rms_e * gk[j];
    __syncthreads();
    double dot = 0.0;  // meaningful in lane 0 of each wave
    for (int i = wave; i < d_model; i += NWAVE) {
      const float* row = wk + (int64_t)i * d_mem;
      double k = 0.0;
      for (int j = lane; j < d_mem; j += 64) k += (double)row[j] * s_en[j];
      k = wave_sum(k);
      dot += ((double)h[i] / rms_h * gq[i]) * k;
    }
    if (lane == 0) s_dot[wave] = dot;
    __syncthreads();
    for (int w = 0; w < NWAVE; ++w) logit += s_dot[w];
  } else {
    // the raw projection k = W_K e into LDS, then its RMSNorm over the d_model features
    double* s_k = s_en + d_mem;
    for (int j = threadIdx.x; j < d_mem; j += NTHR) s_en[j] = e[j];
    __syncthreads();
    for (int i = wave; i < d_model; i += NWAVE) {
      const float* row = wk + (int64_t)i * d_mem;
      double k = 0.0;
      for (int j = lane; j < d_mem; j += 64) k += (double)row[j] * s_en[j];
      k = wave_sum(k);
      if (lane == 0) s_k[i] = k;
    }
    __syncthreads();
    double kk = 0.0, dot = 0.0;
    for (int i = threadIdx.x; i < d_model; i += NTHR) {
      kk += s_k[i] * s_k[i];
      dot += ((double)h[i] / rms_h * gq[i]) * s_k[i] * gk[i];
    }
    const double rms_k = sqrt(block_sum(kk, red) / d_model + eps);
    logit = block_sum(dot, red) / rms_k;
  }
  logit /= sqrt((double)d_model);
  const double alpha = 1.0 / (1.0 + exp(-logit));
  if (threadIdx.x == 0 && a.gate_out != nullptr) a.gate_out[(int64_t)m * a.n_tok + t] = (float)alpha;

  // every thread of the wave holds h[i]; stores happen after the last read of h
  // in this loop iteration, so out may alias h
  for (int i = wave; i < d_model; i += NWAVE) {
    const float* row = wv + (int64_t)i * d_mem;
    double v = 0.0;
    for (int j = lane; j < d_mem; j += 64) v += (double)row[j] * e[j];
    v = wave_sum(v);
    const double hi = h[i];
    if (lane == 0) {
      out[i] = (float)(hi + alpha * v);
      if (vout != nullptr) vout[i] = (float)(alpha * v);
    }
  }
}

}  // namespace

void launch_gate_f32(const GateArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.n_tok, (unsigned)a.n_branch);
  const size_t lds = ((size_t)a.d_mem + (a.key_norm == ENGRAM_KEY_NORM_PROJECTED ? (size_t)a.d_model : 0)) *
                     sizeof(double);
  hipLaunchKernelGGL(gate_f32_kernel, grid, dim3(NTHR), lds, s, a);
}

}  // namespace engram
