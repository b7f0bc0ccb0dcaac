// gate_bf16.hip -- context-aware gating on the gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// "Conditional Memory via Scalable Lookup", section 2.3, Eq. (3)-(4) with the
// gated value and residual update, and section 2.4, Eq. (6) for branches that
// share one memory vector.  Per token t and branch m (key normalised before
// W_K, as in the review page's context_aware_gating pseudocode):
//   k = W_K RMSNorm_gk(e_t),  v = W_V e_t,  q = RMSNorm_gq(h_t)
//   alpha = sigmoid(q . k / sqrt(d_model)),   out_t = h_t + alpha v
//
// The two projections are dense contractions [tokens x d_mem] x [d_mem x d_model]
// and run as bf16 MFMA GEMMs (v_mfma_f32_32x32x16_bf16).  The catch is that
// alpha needs the whole d_model-long dot product q . k before any element of
// the value can be scaled, so the work is split in two launches over the same
// tiling:
//   phase K: acc = W_K' e^T per (feature tile, token tile), W_K' = W_K * diag(gk)
//            (prepared once per call by scale_cols_kernel);  the epilogue
//            reduces  sum_f h[t,f] gq[f] acc[f,t]  and  sum_f h[t,f]^2  over the
//            tile's features into per-(feature tile, token) partials; the main
//            loop also squares one slice of the memory row (k-steps with
//            kt % n_ftiles == ftile) so that the sums of e^2 come for free;
//   phase V: a prologue turns the partials into alpha for the tile's tokens
//            (fixed-order sums, so results are bit-reproducible); the main loop
//            is acc = W_V e^T and the epilogue writes out = h + alpha acc.
// Since  q . k = (sum_f h_f gq_f k~_f) / (rms(h) rms(e))  with k~ = W_K' e, the
// RMSNorm scales are applied to the reduced scalar, never to a tensor.
//
// Tiling: 256 features x 256 tokens per workgroup, BK = 64, four wavefronts in
// a 2 x 2 arrangement, each owning 128 x 128 outputs = 4 x 4 MFMA 32x32 tiles
// (256 fp32 accumulators per lane).  Features are the MFMA rows, so a lane's
// 16 accumulators of one tile belong to ONE token and 4 groups of 4
// consecutive features: the epilogue's h loads and out stores are 8-byte
// vectors, and the per-token reductions are plain adds inside a lane.
// Operands are staged global -> registers -> LDS (double-buffered, one barrier
// per k-step, next k-step's global loads in flight during the MFMAs); LDS rows
// are 128 B with the 16-B chunk index XOR-swizzled by the row.
#include "engram_internal.h"

namespace engram {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int BF = 256;   // features per workgroup
constexpr int BT = 256;   // tokens per workgroup
constexpr int BK = 64;    // contraction depth per k-step
constexpr int NTHR = 256;
constexpr int WF = 128, WT = 128;           // per-wavefront tile
constexpr int MF = WF / 32, MT = WT / 32;   // MFMA tiles per wavefront
constexpr int A_CHUNKS = BF * BK / 8 / NTHR;  // 16-B chunks of the weight tile per thread
constexpr int B_CHUNKS = BT * BK / 8 / NTHR;  // 16-B chunks of the memory tile per thread
constexpr int LDS_A = BF * BK;              // bf16 elements
constexpr int LDS_B = BT * BK;

enum { PHASE_K = 0, PHASE_V = 1 };

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  // round-to-nearest-even conversion (v_cvt_pk_bf16_f32 on gfx950)
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// 16-B chunk position of logical chunk `c` in LDS row `row`
__device__ __forceinline__ int swz(int row, int c) { return c ^ (row & 7); }

__device__ __forceinline__ float sum_sq8(const uint4& v) {
  float s = 0.f;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = bf16_lo(w[i]), b = bf16_hi(w[i]);
    s += a * a;
    s += b * b;
  }
  return s;
}

template <int PHASE>
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gate_mfma_kernel(const GateArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][LDS_A + LDS_B];
  __shared__ float s_red[2][2][BT];  // [wave row][dot, hh][token]
  __shared__ float s_alpha[BT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wf = wave >> 1, wt = wave & 1;
  const int ftile = blockIdx.x;
  const int m = blockIdx.z;
  const int f0 = ftile * BF;
  const int64_t t0 = (int64_t)blockIdx.y * BT;
  const int64_t n_tok = a.n_tok;
  const int d_mem = a.d_mem, d_model = a.d_model;

  // phase K reads the gk-scaled copy of W_K (a.wk points at it here)
  const uint16_t* W = (const uint16_t*)(PHASE == PHASE_K ? a.wk[m] : a.wv[m]);
  const uint16_t* E = (const uint16_t*)a.mem;
  const uint16_t* H = (const uint16_t*)a.h[m];

  // ---- phase V prologue: alpha for this tile's tokens
  if (PHASE == PHASE_V) {
    if (tid < BT) {
      const int64_t t = t0 + tid;
      float alpha = 0.f;
      if (t < n_tok) {
        float dot = 0.f, hh = 0.f, ee = 0.f;
        const int64_t base = (int64_t)m * a.n_ftiles * n_tok + t;
        for (int j = 0; j < a.n_ftiles; ++j) {
          dot += a.part_dot[base + (int64_t)j * n_tok];
          hh += a.part_hh[base + (int64_t)j * n_tok];
          ee += a.ee[base + (int64_t)j * n_tok];
        }
        const float rms_h = sqrtf(hh / (float)d_model + a.eps);
        const float rms_e = sqrtf(ee / (float)d_mem + a.eps);
        const float logit = dot / (rms_h * rms_e) * a.inv_sqrt_d;
        alpha = 1.f / (1.f + expf(-logit));
        if (ftile == 0 && a.gate_out != nullptr) a.gate_out[(int64_t)m * n_tok + t] = alpha;
      }
      s_alpha[tid] = alpha;
    }
  }

  // ---- global -> register staging addresses (row-clamped: padded rows read valid memory)
  const int lrow = tid >> 3;  // + 32 * i
  const int lcc = tid & 7;
  const uint16_t* a_src[A_CHUNKS];
  const uint16_t* b_src[B_CHUNKS];
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) {
    int f = f0 + lrow + 32 * i;
    f = f < d_model ? f : d_model - 1;
    a_src[i] = W + (int64_t)f * d_mem + lcc * 8;
  }
#pragma unroll
  for (int i = 0; i < B_CHUNKS; ++i) {
    int64_t t = t0 + lrow + 32 * i;
    t = t < n_tok ? t : n_tok - 1;
    b_src[i] = E + t * d_mem + lcc * 8;
  }

  uint4 ra[A_CHUNKS], rb[B_CHUNKS];
  float ee_acc[B_CHUNKS];
#pragma unroll
  for (int i = 0; i < B_CHUNKS; ++i) ee_acc[i] = 0.f;

  auto load_global = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + kt * BK);
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + kt * BK);
  };
  auto store_lds = [&](int buf) {
    uint16_t* la = lds[buf];
    uint16_t* lb = lds[buf] + LDS_A;
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int row = lrow + 32 * i;
      *reinterpret_cast<uint4*>(la + row * BK + swz(row, lcc) * 8) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      const int row = lrow + 32 * i;
      *reinterpret_cast<uint4*>(lb + row * BK + swz(row, lcc) * 8) = rb[i];
    }
  };

  floatx16 acc[MF][MT];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = d_mem / BK;
  load_global(0);
  if (PHASE == PHASE_K && (0 % a.n_ftiles) == ftile) {
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) ee_acc[i] += sum_sq8(rb[i]);
  }
  store_lds(0);
  __syncthreads();

  const int arow0 = wf * WF + (lane & 31);
  const int brow0 = wt * WT + (lane & 31);
  const int khalf = lane >> 5;

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) load_global(kt + 1);
    const uint16_t* la = lds[cur];
    const uint16_t* lb = lds[cur] + LDS_A;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int c = s * 2 + khalf;
      bf16x8 af[MF], bfr[MT];
#pragma unroll
      for (int i = 0; i < MF; ++i) {
        const int row = arow0 + i * 32;
        af[i] = *reinterpret_cast<const bf16x8*>(la + row * BK + swz(row, c) * 8);
      }
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const int row = brow0 + j * 32;
        bfr[j] = *reinterpret_cast<const bf16x8*>(lb + row * BK + swz(row, c) * 8);
      }
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < MT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      if (PHASE == PHASE_K && ((kt + 1) % a.n_ftiles) == ftile) {
#pragma unroll
        for (int i = 0; i < B_CHUNKS; ++i) ee_acc[i] += sum_sq8(rb[i]);
      }
      store_lds(cur ^ 1);
    }
    __syncthreads();
  }

  // ---- epilogues.  Lane owns token column (lane & 31) of every MFMA tile and
  // features 8*g + 4*(lane >> 5) + {0..3} of it (g = 0..3).
  const int fl = (lane >> 5) * 4;
  if (PHASE == PHASE_K) {
    // sums of e^2 over this block's slice of the memory row
    float* ee_out = a.ee + ((int64_t)m * a.n_ftiles + ftile) * n_tok;
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      float v = ee_acc[i];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      const int64_t t = t0 + lrow + 32 * i;
      if (lcc == 0 && t < n_tok) ee_out[t] = v;
    }
    const uint16_t* GQ = (const uint16_t*)a.gq[m];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int tl = wt * WT + j * 32 + (lane & 31);
      const int64_t t = t0 + tl;
      float dot = 0.f, hh = 0.f;
      if (t < n_tok) {
        const uint16_t* hrow = H + t * d_model;
#pragma unroll
        for (int i = 0; i < MF; ++i) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int f = f0 + wf * WF + i * 32 + g * 8 + fl;
            if (f < d_model) {
              const uint2 hv = *reinterpret_cast<const uint2*>(hrow + f);
              const uint2 gv = *reinterpret_cast<const uint2*>(GQ + f);
              const float h0 = bf16_lo(hv.x), h1 = bf16_hi(hv.x), h2 = bf16_lo(hv.y), h3 = bf16_hi(hv.y);
              dot += h0 * bf16_lo(gv.x) * acc[i][j][g * 4 + 0];
              dot += h1 * bf16_hi(gv.x) * acc[i][j][g * 4 + 1];
              dot += h2 * bf16_lo(gv.y) * acc[i][j][g * 4 + 2];
              dot += h3 * bf16_hi(gv.y) * acc[i][j][g * 4 + 3];
              hh += h0 * h0 + h1 * h1 + h2 * h2 + h3 * h3;
            }
          }
        }
      }
      dot += __shfl_xor(dot, 32, 64);
      hh += __shfl_xor(hh, 32, 64);
      if (lane < 32) {
        s_red[wf][0][tl] = dot;
        s_red[wf][1][tl] = hh;
      }
    }
    __syncthreads();
    if (tid < BT) {
      const int64_t t = t0 + tid;
      if (t < n_tok) {
        const int64_t o = ((int64_t)m * a.n_ftiles + ftile) * n_tok + t;
        a.part_dot[o] = s_red[0][0][tid] + s_red[1][0][tid];
        a.part_hh[o] = s_red[0][1][tid] + s_red[1][1][tid];
      }
    }
  } else {
    uint16_t* O = (uint16_t*)a.out[m];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int tl = wt * WT + j * 32 + (lane & 31);
      const int64_t t = t0 + tl;
      if (t >= n_tok) continue;
      const float alpha = s_alpha[tl];
      const uint16_t* hrow = H + t * d_model;
      uint16_t* orow = O + t * d_model;
#pragma unroll
      for (int i = 0; i < MF; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int f = f0 + wf * WF + i * 32 + g * 8 + fl;
          if (f < d_model) {
            const uint2 hv = *reinterpret_cast<const uint2*>(hrow + f);
            uint2 o;
            o.x = pack_bf16(bf16_lo(hv.x) + alpha * acc[i][j][g * 4 + 0],
                            bf16_hi(hv.x) + alpha * acc[i][j][g * 4 + 1]);
            o.y = pack_bf16(bf16_lo(hv.y) + alpha * acc[i][j][g * 4 + 2],
                            bf16_hi(hv.y) + alpha * acc[i][j][g * 4 + 3]);
            *reinterpret_cast<uint2*>(orow + f) = o;
          }
        }
      }
    }
  }
}

// W'[i][j] = bf16(W[i][j] * g[j]) for the key projection of one branch.
__global__ __launch_bounds__(256) void scale_cols_kernel(const uint16_t* __restrict__ w,
                                                         const uint16_t* __restrict__ g,
                                                         uint16_t* __restrict__ out, int64_t n8,
                                                         int d_mem) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const int j = (int)((i * 8) % d_mem);
  const uint4 wv = reinterpret_cast<const uint4*>(w)[i];
  const uint4 gv = *reinterpret_cast<const uint4*>(g + j);
  uint4 o;
  o.x = pack_bf16(bf16_lo(wv.x) * bf16_lo(gv.x), bf16_hi(wv.x) * bf16_hi(gv.x));
  o.y = pack_bf16(bf16_lo(wv.y) * bf16_lo(gv.y), bf16_hi(wv.y) * bf16_hi(gv.y));
  o.z = pack_bf16(bf16_lo(wv.z) * bf16_lo(gv.z), bf16_hi(wv.z) * bf16_hi(gv.z));
  o.w = pack_bf16(bf16_lo(wv.w) * bf16_lo(gv.w), bf16_hi(wv.w) * bf16_hi(gv.w));
  reinterpret_cast<uint4*>(out)[i] = o;
}

struct ScratchLayout {
  size_t wk_bytes, part_elems, total;
};

ScratchLayout layout_for(const GateArgs& a) {
  ScratchLayout L;
  L.wk_bytes = (size_t)a.n_branch * a.d_model * a.d_mem * 2;
  L.wk_bytes = (L.wk_bytes + 255) & ~(size_t)255;
  L.part_elems = (size_t)a.n_branch * a.n_ftiles * (size_t)a.n_tok;
  const size_t part_bytes = ((L.part_elems * 4) + 255) & ~(size_t)255;
  L.total = L.wk_bytes + 3 * part_bytes;
  return L;
}

}  // namespace

size_t gate_bf16_scratch_bytes(GateArgs& a) {
  a.n_ftiles = (a.d_model + BF - 1) / BF;
  return layout_for(a).total;
}

// `a.part_dot` must point at the scratch block of gate_bf16_scratch_bytes(a) bytes;
// the other scratch pointers are carved from it here.
void launch_gate_bf16(const GateArgs& a_in, hipStream_t s) {
  GateArgs a = a_in;
  const ScratchLayout L = layout_for(a);
  char* base = (char*)a_in.part_dot;
  const size_t part_bytes = ((L.part_elems * 4) + 255) & ~(size_t)255;
  for (int m = 0; m < a.n_branch; ++m) {
    uint16_t* dst = (uint16_t*)(base + (size_t)m * a.d_model * a.d_mem * 2);
    const int64_t n8 = (int64_t)a.d_model * a.d_mem / 8;
    hipLaunchKernelGGL(scale_cols_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                       (const uint16_t*)a.wk[m], (const uint16_t*)a.gk[m], dst, n8, a.d_mem);
    a.wk[m] = dst;
  }
  a.part_dot = (float*)(base + L.wk_bytes);
  a.part_hh = (float*)(base + L.wk_bytes + part_bytes);
  a.ee = (float*)(base + L.wk_bytes + 2 * part_bytes);

  const dim3 grid((unsigned)a.n_ftiles, (unsigned)((a.n_tok + BT - 1) / BT), (unsigned)a.n_branch);
  hipLaunchKernelGGL(gate_mfma_kernel<PHASE_K>, grid, dim3(NTHR), 0, s, a);
  hipLaunchKernelGGL(gate_mfma_kernel<PHASE_V>, grid, dim3(NTHR), 0, s, a);
}

}  // namespace engram
