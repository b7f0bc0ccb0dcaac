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
// and run as bf16 MFMA GEMMs (v_mfma_f32_32x32x16_bf16).  alpha needs the whole
// d_model-long dot product q . k before any element of the value can be scaled,
// so the work is two launches over the same tiling:
//   phase K: acc = W_K' e^T per (feature tile, token tile), W_K' = W_K diag(gk)
//            (prepared once per call by scale_cols_kernel); the epilogue reduces
//            sum_f h[t,f] gq[f] acc[f,t] and sum_f h[t,f]^2 over the tile's
//            features into per-(feature tile, token) partials; the main loop
//            also sums e^2 over one slice of the memory row (k-steps with
//            kt % n_ftiles == ftile), so every tile does 1/n_ftiles of it;
//   phase V: a prologue turns the partials into alpha for the tile's tokens
//            (fixed-order sums, bit-reproducible); the main loop is
//            acc = W_V e^T and the epilogue writes out = h + alpha acc.
// Since q . k = (sum_f h_f gq_f k~_f) / (rms(h) rms(e)) with k~ = W_K' e, the
// RMSNorm scales are applied to the reduced scalar, never to a tensor.
//
// Tiling.  256 features x 256 tokens per workgroup, four wavefronts in 2 x 2,
// each owning 128 x 128 outputs = 4 x 4 MFMA 32x32 tiles (256 fp32
// accumulators per lane).  Features are the MFMA rows, so all 16 accumulators
// of a lane in one tile belong to ONE token; the weight rows are loaded in a
// permuted order (bits 2 and 3 of the row index swapped inside each 32-row
// tile) so that a lane's accumulator groups 0-1 and 2-3 each cover 8
// consecutive features: every epilogue access is a 16-byte vector.
//
// Main loop.  BK = 64 per k-step, double-buffered LDS (2 x 64 KB).  The next
// k-step's operands are loaded global -> registers (16-B native vectors, so the
// staging array stays in registers) while the current k-step's 64 MFMAs run,
// then written to the other LDS buffer; one LDS-only barrier per k-step (a
// plain __syncthreads() would also wait for the in-flight global loads).
// LDS rows are 128 B; the 16-B chunk index is XOR-swizzled with
// (r & 7) ^ ((r >> 3) & 1), which keeps the fragment reads (32 consecutive
// rows, one chunk) free of bank conflicts for 128- and 256-byte LDS clocks.
//
// Epilogue.  The LDS buffers are reused for the h tile (256 tokens x 256
// features, 128 KB), loaded with coalesced 16-byte loads; 16-byte chunks
// are swizzled by (token & 31) so that 32 lanes reading 32 tokens hit distinct
// banks.  Phase V writes out into the same LDS tile and then streams it to
// HBM with coalesced 16-byte stores.
#include <type_traits>

#include "engram_internal.h"

namespace engram {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16-B chunk (native vector: stays in registers)

constexpr int BF = 256;   // features per workgroup
constexpr int BT = 256;   // tokens per workgroup
constexpr int BK = 64;    // contraction depth per stage
constexpr int NSTAGE = 2;  // LDS double buffer
constexpr int NTHR = 256;
constexpr int WF = 128, WT = 128;           // per-wavefront tile
constexpr int MF = WF / 32, MT = WT / 32;   // MFMA tiles per wavefront
constexpr int ROW_CH = BK / 8;              // 16-B chunks per LDS row (8)
constexpr int STAGE_A = BF * BK;            // bf16 elements of the weight tile in a stage
constexpr int STAGE = (BF + BT) * BK;       // bf16 elements per stage
constexpr int CH_A = BF * ROW_CH / NTHR;   // 16-B chunks of the weight tile per thread per stage
constexpr int CH_B = BT * ROW_CH / NTHR;   // 16-B chunks of the memory tile per thread per stage
constexpr int H_CH = BF / 8;               // 16-B chunks per h row in the epilogue tile (32)
constexpr int H_LOADS = BT * H_CH / NTHR;  // 32 chunks per thread
constexpr int SMEM_ELEMS = (NSTAGE * STAGE > BT * BF) ? NSTAGE * STAGE : BT * BF;

enum { PHASE_K = 0, PHASE_V = 1 };

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  // round-to-nearest-even conversion (v_cvt_pk_bf16_f32 on gfx950)
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Physical 16-B chunk of logical chunk c in a 128-B stage row r.  Fragment reads
// hit 32 consecutive rows at one logical chunk; (r & 7) ^ ((r >> 3) & 1) keeps
// them conflict-free whether the LDS serves 128 or 256 bytes per clock.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r & 7) ^ ((r >> 3) & 1)); }
// LDS element offset of 16-B chunk q (row q / ROW_CH) of a stage operand tile
__device__ __forceinline__ int st_off(int q) {
  const int r = q / ROW_CH;
  return r * BK + swz(r, q % ROW_CH) * 8;
}
// feature offset (inside a 32-row MFMA tile) held by MFMA row rho: bits 2 and 3 swapped
__device__ __forceinline__ int tile_row_feature(int rho) {
  return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads() it does
// not wait for this wave's in-flight global loads (the next stages' prefetch).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float sumsq8(const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float s = 0.f;
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
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM_ELEMS];  // stage ring, then h tile
  __shared__ float s_red[2][2][BT];  // [feature-wave][dot, hh][token]
  __shared__ float s_alpha[BT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wf = wave >> 1, wt = wave & 1;

  // ---- XCD-aware tile order: hardware block b runs on XCD b % 8; give each XCD a
  // contiguous run of logical tiles (feature tile fastest, so an XCD's concurrent
  // blocks share memory-vector tiles in its L2)
  const int n_ttiles = (int)((a.n_tok + BT - 1) / BT);
  const uint32_t nblocks = gridDim.x;
  uint32_t logical = blockIdx.x;
  if ((nblocks & 7) == 0) logical = (blockIdx.x & 7) * (nblocks >> 3) + (blockIdx.x >> 3);
  const int ftile = (int)(logical % (uint32_t)a.n_ftiles);
  const uint32_t rest = logical / (uint32_t)a.n_ftiles;
  const int ttile = (int)(rest % (uint32_t)n_ttiles);
  const int m = (int)(rest / (uint32_t)n_ttiles);

  const int f0 = ftile * BF;
  const int64_t t0 = (int64_t)ttile * BT;
  const int64_t n_tok = a.n_tok;
  const int d_mem = a.d_mem, d_model = a.d_model;

  // phase K reads the gk-scaled copy of W_K (a.wk points at it here)
  const uint16_t* W = (const uint16_t*)(PHASE == PHASE_K ? a.wk[m] : a.wv[m]);
  const uint16_t* E = (const uint16_t*)a.mem;
  const uint16_t* H = (const uint16_t*)a.h[m];

  // ---- phase V prologue: alpha for this tile's tokens
  if (PHASE == PHASE_V) {
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

  // ---- global -> register -> LDS staging.  Thread tid moves 16-B chunks
  // q = tid + NTHR * i of each operand tile: row q / ROW_CH, logical chunk q % ROW_CH.
  // All offsets are 32-bit from wave-uniform bases, so the loads take the
  // scalar-base + vector-offset form and only one VGPR per chunk stays live.
  const uint16_t* Et0 = E + t0 * d_mem;   // memory rows of this token tile
  uint32_t a_off[CH_A], b_off[CH_B];
#pragma unroll
  for (int i = 0; i < CH_A; ++i) {
    const int q = tid + NTHR * i;
    const int r = q / ROW_CH, c = q % ROW_CH;
    int f = f0 + (r & ~31) + tile_row_feature(r & 31);
    f = f < d_model ? f : d_model - 1;   // rows past d_model: any valid row, result unused
    a_off[i] = (uint32_t)f * (uint32_t)d_mem + c * 8;
  }
#pragma unroll
  for (int i = 0; i < CH_B; ++i) {
    const int q = tid + NTHR * i;
    const int r = q / ROW_CH, c = q % ROW_CH;
    const int rr = t0 + r < n_tok ? r : (int)(n_tok - 1 - t0);  // padded tokens: a valid row
    b_off[i] = (uint32_t)rr * (uint32_t)d_mem + c * 8;
  }


  u32x4 ra[CH_A], rb[CH_B];  // the next stage, in flight while the current one is consumed
#define ENGRAM_LOAD_STAGE(kt)                                                              \
  do {                                                                                     \
    const int k0_ = (kt) * BK;                                                             \
    _Pragma("unroll") for (int i = 0; i < CH_A; ++i)                                       \
        ra[i] = *reinterpret_cast<const u32x4*>(W + a_off[i] + k0_);                       \
    _Pragma("unroll") for (int i = 0; i < CH_B; ++i)                                       \
        rb[i] = *reinterpret_cast<const u32x4*>(Et0 + b_off[i] + k0_);                     \
  } while (0)
#define ENGRAM_STORE_STAGE(kt)                                                             \
  do {                                                                                     \
    uint16_t* st_ = smem + ((kt) & 1) * STAGE;                                             \
    _Pragma("unroll") for (int i = 0; i < CH_A; ++i)                                       \
        *reinterpret_cast<u32x4*>(st_ + st_off(tid + NTHR * i)) = ra[i];                   \
    _Pragma("unroll") for (int i = 0; i < CH_B; ++i)                                       \
        *reinterpret_cast<u32x4*>(st_ + STAGE_A + st_off(tid + NTHR * i)) = rb[i];         \
  } while (0)

  floatx16 acc[MF][MT];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = d_mem / BK;
  ENGRAM_LOAD_STAGE(0);
  ENGRAM_STORE_STAGE(0);
  lds_barrier();

  const int arow0 = wf * WF + (lane & 31);
  const int brow0 = wt * WT + (lane & 31);
  const int khalf = lane >> 5;
  float ee_acc = 0.f;  // phase K: sum of e^2 of token row `tid` over this tile's k slice

  for (int kt = 0; kt < nk; ++kt) {
    // next stage's global loads fly during this stage's MFMAs
    if (kt + 1 < nk) ENGRAM_LOAD_STAGE(kt + 1);
    const uint16_t* la = smem + (kt & 1) * STAGE;
    const uint16_t* lb = la + STAGE_A;
    if (PHASE == PHASE_K && (kt % a.n_ftiles) == ftile) {
#pragma unroll
      for (int c = 0; c < ROW_CH; ++c)
        ee_acc += sumsq8(*reinterpret_cast<const uint4*>(lb + tid * BK + c * 8));
    }
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int c = s * 2 + khalf;
      bf16x8 af[MF], bfr[MT];
#pragma unroll
      for (int i = 0; i < MF; ++i) {
        const int r = arow0 + i * 32;
        af[i] = *reinterpret_cast<const bf16x8*>(la + r * BK + swz(r, c) * 8);
      }
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const int r = brow0 + j * 32;
        bfr[j] = *reinterpret_cast<const bf16x8*>(lb + r * BK + swz(r, c) * 8);
      }
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < MT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    // the other buffer was last read in k-step kt-1, which every wave finished
    // before the previous barrier
    if (kt + 1 < nk) ENGRAM_STORE_STAGE(kt + 1);
    lds_barrier();
  }
#undef ENGRAM_LOAD_STAGE
#undef ENGRAM_STORE_STAGE

  // Everything below re-derives its indices from an opaque copy of the thread id, so
  // the compiler cannot compute epilogue addresses before the loop and keep them
  // live (in registers the main loop needs) across it.
  int etid = tid;
  asm volatile("" : "+v"(etid));
  const int elane = etid & 63, ewave = etid >> 6;
  const int ewf = ewave >> 1, ewt = ewave & 1;

  if (PHASE == PHASE_K) {
    const int64_t t = t0 + etid;
    if (t < n_tok) a.ee[((int64_t)m * a.n_ftiles + ftile) * n_tok + t] = ee_acc;
  }

  // ---- h tile [BT tokens][BF features] into LDS (16-B chunks swizzled by token);
  // the last loop barrier already retired every read of the stage ring
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    uint4 hv[H_LOADS / 2];
#pragma unroll
    for (int i = 0; i < H_LOADS / 2; ++i) {
      const int p = (half * (H_LOADS / 2) + i) * NTHR + etid;
      const int tl = p / H_CH;
      const int c = (p % H_CH) ^ (tl & 31);
      int64_t t = t0 + tl;
      t = t < n_tok ? t : n_tok - 1;
      int f = f0 + c * 8;
      f = f < d_model ? f : 0;
      hv[i] = *reinterpret_cast<const uint4*>(H + t * d_model + f);
    }
#pragma unroll
    for (int i = 0; i < H_LOADS / 2; ++i) {
      const int p = (half * (H_LOADS / 2) + i) * NTHR + etid;
      *reinterpret_cast<uint4*>(smem + p * 8) = hv[i];
    }
  }
  __syncthreads();

  // Lane (token column tl) holds, for MFMA tile (i, j) and pair gp, features
  // fl = ewf*WF + i*32 + gp*16 + (elane>>5)*8 + 0..7 in acc[i][j][8*gp + 0..7].
  const int hsel = (elane >> 5) * 8;
  if (PHASE == PHASE_K) {
    const uint16_t* GQ = (const uint16_t*)a.gq[m];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int tl = ewt * WT + j * 32 + (elane & 31);
      float dot = 0.f, hh = 0.f;
#pragma unroll
      for (int i = 0; i < MF; ++i) {
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          const int fl = ewf * WF + i * 32 + gp * 16 + hsel;
          if (f0 + fl < d_model) {
            const int c = (fl >> 3) ^ (tl & 31);
            const uint4 hv = *reinterpret_cast<const uint4*>(smem + tl * BF + c * 8);
            const uint4 gv = *reinterpret_cast<const uint4*>(GQ + f0 + fl);
            const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
            const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float h0 = bf16_lo(hw[q]), h1 = bf16_hi(hw[q]);
              dot += h0 * bf16_lo(gw[q]) * acc[i][j][gp * 8 + 2 * q];
              dot += h1 * bf16_hi(gw[q]) * acc[i][j][gp * 8 + 2 * q + 1];
              hh += h0 * h0 + h1 * h1;
            }
          }
        }
      }
      dot += __shfl_xor(dot, 32, 64);
      hh += __shfl_xor(hh, 32, 64);
      if (elane < 32) {
        s_red[ewf][0][tl] = dot;
        s_red[ewf][1][tl] = hh;
      }
    }
    __syncthreads();
    const int64_t t = t0 + etid;
    if (t < n_tok) {
      const int64_t o = ((int64_t)m * a.n_ftiles + ftile) * n_tok + t;
      a.part_dot[o] = s_red[0][0][etid] + s_red[1][0][etid];
      a.part_hh[o] = s_red[0][1][etid] + s_red[1][1][etid];
    }
  } else {
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int tl = ewt * WT + j * 32 + (elane & 31);
      const float alpha = s_alpha[tl];
#pragma unroll
      for (int i = 0; i < MF; ++i) {
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          const int fl = ewf * WF + i * 32 + gp * 16 + hsel;
          const int c = (fl >> 3) ^ (tl & 31);
          uint4* cell = reinterpret_cast<uint4*>(smem + tl * BF + c * 8);
          const uint4 hv = *cell;
          const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
          uint32_t ow[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            ow[q] = pack_bf16(bf16_lo(hw[q]) + alpha * acc[i][j][gp * 8 + 2 * q],
                              bf16_hi(hw[q]) + alpha * acc[i][j][gp * 8 + 2 * q + 1]);
          *cell = make_uint4(ow[0], ow[1], ow[2], ow[3]);
        }
      }
    }
    __syncthreads();
    uint16_t* O = (uint16_t*)a.out[m];
#pragma unroll 4
    for (int i = 0; i < BT * H_CH / NTHR; ++i) {
      const int p = i * NTHR + etid;
      const int tl = p / H_CH;
      const int phys = p % H_CH;
      const int c = phys ^ (tl & 31);
      const int64_t t = t0 + tl;
      const int f = f0 + c * 8;
      if (t < n_tok && f < d_model)
        *reinterpret_cast<uint4*>(O + t * d_model + f) =
            *reinterpret_cast<const uint4*>(smem + tl * BF + phys * 8);
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
  size_t wk_bytes, part_bytes, total;
};

ScratchLayout layout_for(const GateArgs& a) {
  ScratchLayout L;
  L.wk_bytes = ((size_t)a.n_branch * a.d_model * a.d_mem * 2 + 255) & ~(size_t)255;
  const size_t part_elems = (size_t)a.n_branch * a.n_ftiles * (size_t)a.n_tok;
  L.part_bytes = (part_elems * 4 + 255) & ~(size_t)255;
  L.total = L.wk_bytes + 3 * L.part_bytes;
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
  for (int m = 0; m < a.n_branch; ++m) {
    uint16_t* dst = (uint16_t*)(base + (size_t)m * a.d_model * a.d_mem * 2);
    const int64_t n8 = (int64_t)a.d_model * a.d_mem / 8;
    hipLaunchKernelGGL(scale_cols_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                       (const uint16_t*)a.wk[m], (const uint16_t*)a.gk[m], dst, n8, a.d_mem);
    a.wk[m] = dst;
  }
  a.part_dot = (float*)(base + L.wk_bytes);
  a.part_hh = (float*)(base + L.wk_bytes + L.part_bytes);
  a.ee = (float*)(base + L.wk_bytes + 2 * L.part_bytes);

  const int64_t n_ttiles = (a.n_tok + BT - 1) / BT;
  const unsigned blocks = (unsigned)(n_ttiles * a.n_ftiles * a.n_branch);
  hipLaunchKernelGGL(gate_mfma_kernel<PHASE_K>, dim3(blocks), dim3(NTHR), 0, s, a);
  hipLaunchKernelGGL(gate_mfma_kernel<PHASE_V>, dim3(blocks), dim3(NTHR), 0, s, a);
}

}  // namespace engram
