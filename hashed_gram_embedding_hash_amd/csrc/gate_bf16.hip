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
// so every output tile is computed twice over the same tiling:
//   K tile: acc = W_K' e^T for (feature tile, token tile), W_K' = W_K diag(gk)
//           (prepared once per call by gate_prep_kernel); the epilogue reduces
//           sum_f h[t,f] gq[f] acc[f,t] and sum_f h[t,f]^2 over the tile's
//           features into per-(feature tile, token) partials; the main loop
//           also sums e^2 over one slice of the memory row (k-steps with
//           kt % n_ftiles == ftile), so every tile does 1/n_ftiles of it;
//   V tile: waits until all K tiles of its (branch, token tile) are done,
//           turns the partials into alpha (fixed-order sums: bit-reproducible),
//           computes acc = W_V e^T and writes out = h + alpha acc.
// Since q . k = (sum_f h_f gq_f k~_f) / (rms(h) rms(e)) with k~ = W_K' e, the
// RMSNorm scales are applied to the reduced scalar, never to a tensor.
//
// Scheduling.  One persistent launch of one workgroup per CU.  Workgroup b
// serves work queue b % 8 (the XCD it is dispatched to), which holds the token
// tiles T with T % 8 == b % 8: first all their K tiles, then all their V tiles,
// feature tile fastest.  A workgroup claims the next tile of its queue with an
// atomic increment; a V tile spins until the done-counter of its K tiles is
// full.  Those K tiles sit earlier in the same queue, so they were claimed
// before by running workgroups that never wait: the spin always ends.  The
// single queue per XCD removes the partial last round of a two-launch design
// (640 + 640 tiles on 256 CUs become 1280 = 5 x 256) and keeps a token tile's
// memory rows in one XCD's L2.
//
// Tiling.  256 features x 256 tokens per tile, four wavefronts in 2 x 2, each
// owning 128 x 128 outputs = 4 x 4 MFMA 32x32 tiles (256 fp32 accumulators per
// lane).  Features are the MFMA rows, so all 16 accumulators of a lane in one
// MFMA tile belong to ONE token; weight rows are loaded in a permuted order
// (bits 2 and 3 of the row index swapped inside each 32-row tile) so that a
// lane's accumulator groups 0-1 and 2-3 each cover 8 consecutive features:
// every epilogue access is a 16-byte vector.
//
// Main loop.  BK = 64 per k-step, double-buffered LDS (2 x 64 KB).  The next
// k-step's operands are loaded global -> registers (16-B native vectors, so the
// staging array stays in registers) while the current k-step's 64 MFMAs run,
// then written to the other LDS buffer; one LDS-only barrier per k-step (a
// plain __syncthreads() would also wait for the in-flight global loads).  The
// loop body is branch-free; the fragment registers are double-buffered so the
// LDS reads of sub-step s+1 are in flight during sub-step s's MFMAs.  LDS rows are 128 B; the 16-B chunk index is XOR-swizzled with
// (r & 7) ^ ((r >> 3) & 1), which keeps the fragment reads (32 consecutive
// rows, one chunk) free of bank conflicts.
//
// Epilogue.  The LDS buffers are reused for the h tile (256 tokens x 256
// features, 128 KB), loaded with coalesced 16-byte loads; 16-byte chunks
// are swizzled by (token & 31) so that 32 lanes reading 32 tokens hit distinct
// banks.  A V tile writes out into the same LDS tile and then streams it to
// HBM with coalesced 16-byte stores.
#include "engram_internal.h"

namespace engram {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16-B chunk (native: stays in registers)

constexpr int BF = 256;   // features per tile
constexpr int BT = 256;   // tokens per tile
constexpr int BK = 64;    // contraction depth per k-step
constexpr int NTHR = 256;
constexpr int WF = 128, WT = 128;           // per-wavefront tile
constexpr int MF = WF / 32, MT = WT / 32;   // MFMA tiles per wavefront
constexpr int ROW_CH = BK / 8;              // 16-B chunks per LDS row (8)
constexpr int STAGE_A = BF * BK;            // bf16 elements of the weight tile in a stage
constexpr int STAGE = (BF + BT) * BK;       // bf16 elements per stage
constexpr int CH_A = BF * ROW_CH / NTHR;    // 16-B chunks of the weight tile per thread per stage
constexpr int CH_B = BT * ROW_CH / NTHR;    // 16-B chunks of the memory tile per thread per stage
constexpr int H_CH = BF / 8;                // 16-B chunks per h row in the epilogue tile (32)
constexpr int H_LOADS = BT * H_CH / NTHR;   // 32 chunks per thread
constexpr int SMEM_ELEMS = (2 * STAGE > BT * BF) ? 2 * STAGE : BT * BF;
constexpr int NQ = 8;                       // work queues (one per XCD)
constexpr int SPIN_LIMIT = 1 << 24;         // ~0.5 s of s_sleep before a V tile gives up waiting

enum { PHASE_K = 0, PHASE_V = 1 };

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  // round-to-nearest-even conversion (v_cvt_pk_bf16_f32 on gfx950)
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Physical 16-B chunk of logical chunk c in a 128-B stage row r.
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

__device__ __forceinline__ float sumsq8(const u32x4& v) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = bf16_lo(v[i]), b = bf16_hi(v[i]);
    s += a * a;
    s += b * b;
  }
  return s;
}

// Partials cross workgroups (K tiles write, V tiles of the same token tile read).
// They travel as device-coherent relaxed atomic stores/loads, which are performed
// at the device coherence point without flushing or invalidating whole caches; the
// done counter is incremented only after the writers' stores completed (workgroup
// barrier), and a reader issues its loads only after it saw the full count.
// Full acquire/release at device scope would write back and invalidate the XCD's
// L2 on every tile, evicting the operand tiles the other CUs are streaming.
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Half `half` (tokens 128 half .. 128 half + 127) of the epilogue's h tile
// [BT tokens][BF features] straight into LDS with direct global->LDS loads: LDS
// 16-B chunk P = tl * 32 + phys holds logical chunk phys ^ (tl & 31) of token tl
// (the swizzle keeps the epilogue's 32-tokens-per-read accesses conflict-free).
// Every wave instruction fills 64 consecutive chunks (two token rows).
__device__ __forceinline__ void load_h_half(uint16_t* smem, const uint16_t* Ht0, int64_t t0,
                                            int64_t n_tok, int f0, int d_model, int half,
                                            int wave, int lane) {
  typedef __attribute__((address_space(3))) void lds_void;
  const int tr_lim = (int)(n_tok - 1 - t0);
#pragma unroll
  for (int i = 0; i < H_LOADS / 2; ++i) {
    const int base = half * (BT / 2) * H_CH + (wave * (H_LOADS / 2) + i) * 64;  // wave-uniform
    const int p = base + lane;
    const int tl = p / H_CH;
    const int c = (p % H_CH) ^ (tl & 31);
    const int tr = tl < tr_lim ? tl : tr_lim;   // tokens past n_tok: a valid row, unused
    int f = f0 + c * 8;
    f = f < d_model ? f : 0;
    __builtin_amdgcn_global_load_lds(Ht0 + (uint32_t)tr * (uint32_t)d_model + f,
                                     (lds_void*)(smem + base * 8), 16, 0, 0);
  }
}

struct Tile {
  int phase, m, ttile, ftile;
};

// Tile q of queue x; false once the queue is exhausted.
__device__ __forceinline__ bool decode_tile(const GateArgs& a, int x, int q, Tile& t) {
  const int n_tt = a.n_ttiles > x ? (a.n_ttiles - x + NQ - 1) / NQ : 0;  // token tiles of queue x
  const int per_tt = a.n_branch * a.n_ftiles;
  const int per_phase = n_tt * per_tt;
  if (q >= 2 * per_phase) return false;
  t.phase = q >= per_phase ? PHASE_V : PHASE_K;
  const int r = q - t.phase * per_phase;
  const int tl = r / per_tt;
  const int r2 = r - tl * per_tt;
  t.m = r2 / a.n_ftiles;
  t.ftile = r2 - t.m * a.n_ftiles;
  t.ttile = tl * NQ + x;
  return true;
}

// One K or V tile.  A single main loop serves both phases (one copy of the
// loop keeps register allocation simple); only the epilogues differ.
__device__ __forceinline__ void gate_tile(const GateArgs& a, const Tile& tile, uint16_t* smem,
                                          float (*s_red)[2][BT], float* s_alpha) {
  const int PHASE = tile.phase;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wf = wave >> 1, wt = wave & 1;
  const int m = tile.m, ftile = tile.ftile;
  const int f0 = ftile * BF;
  const int64_t t0 = (int64_t)tile.ttile * BT;
  const int64_t n_tok = a.n_tok;
  const int d_mem = a.d_mem, d_model = a.d_model;
  int32_t* done = a.counters + NQ + m * a.n_ttiles + tile.ttile;

  // phase K reads the gk-scaled copy of W_K (a.wk points at it here)
  const uint16_t* W = (const uint16_t*)(PHASE == PHASE_K ? a.wk[m] : a.wv[m]);
  const uint16_t* E = (const uint16_t*)a.mem;
  const uint16_t* H = (const uint16_t*)a.h[m];

  if (PHASE == PHASE_V) {
    // ---- wait for the K tiles of this (branch, token tile), then alpha per token
    if (tid == 0) {
      int spin = 0;
      while (__hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < a.n_ftiles &&
             ++spin < SPIN_LIMIT)
        __builtin_amdgcn_s_sleep(1);
    }
    __syncthreads();  // the partial loads below are issued only after the count is seen
    const int64_t t = t0 + tid;
    float alpha = 0.f;
    if (t < n_tok) {
      float dot = 0.f, hh = 0.f, ee = 0.f;
      const int64_t base = (int64_t)m * a.n_ftiles * n_tok + t;
      for (int j = 0; j < a.n_ftiles; ++j) {
        dot += ld_coherent(a.part_dot + base + (int64_t)j * n_tok);
        hh += ld_coherent(a.part_hh + base + (int64_t)j * n_tok);
        ee += ld_coherent(a.ee + base + (int64_t)j * n_tok);
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
  // Offsets are 32-bit from wave-uniform bases.
  const uint16_t* Et0 = E + t0 * d_mem;  // memory rows of this token tile
  // Chunk i of this thread sits in row (tid / ROW_CH) + 32 i, logical chunk tid % ROW_CH.
  // The weight row permutation only touches the low 5 bits of the row, so row i of the
  // weight tile is feature f0 + 32 i + tile_row_feature(tid / ROW_CH); rows past d_model
  // (and tokens past n_tok) are clamped to a valid row whose result is unused.
  const int srow = tid / ROW_CH;                     // 0..31
  const int scol = (tid % ROW_CH) * 8;
  const int a_f = f0 + tile_row_feature(srow);
  const int b_lim = (int)(n_tok - 1 - t0);           // last valid row of the token tile
#define ENGRAM_A_OFF(i) ((uint32_t)min(a_f + 32 * (i), d_model - 1) * (uint32_t)d_mem + scol)
#define ENGRAM_B_OFF(i) ((uint32_t)min(srow + 32 * (i), b_lim) * (uint32_t)d_mem + scol)

  // The next stage's global loads, in flight in registers across a k-step's MFMAs.
  // Native 16-byte vectors with static indices keep them out of scratch.
  u32x4 ra[CH_A], rb[CH_B];
#define ENGRAM_LOAD_STAGE(kt)                                                              \
  do {                                                                                     \
    const int k0_ = (kt) * BK;                                                             \
    _Pragma("unroll") for (int i = 0; i < CH_A; ++i)                                       \
        ra[i] = *reinterpret_cast<const u32x4*>(W + ENGRAM_A_OFF(i) + k0_);                \
    _Pragma("unroll") for (int i = 0; i < CH_B; ++i)                                       \
        rb[i] = *reinterpret_cast<const u32x4*>(Et0 + ENGRAM_B_OFF(i) + k0_);              \
  } while (0)
#define ENGRAM_STORE_STAGE(buf)                                                            \
  do {                                                                                     \
    uint16_t* st_ = smem + (buf) * STAGE;                                                  \
    _Pragma("unroll") for (int i = 0; i < CH_A; ++i)                                       \
        *reinterpret_cast<u32x4*>(st_ + st_off(tid + NTHR * i)) = ra[i];                   \
    _Pragma("unroll") for (int i = 0; i < CH_B; ++i)                                       \
        *reinterpret_cast<u32x4*>(st_ + STAGE_A + st_off(tid + NTHR * i)) = rb[i];         \
  } while (0)
  // sums of e^2 of the rows this thread stages (rows tid / ROW_CH + 32 i), over the
  // k-steps of this tile's slice
  float ee_rows[CH_B];
#pragma unroll
  for (int i = 0; i < CH_B; ++i) ee_rows[i] = 0.f;
#define ENGRAM_EE(kt_stage)                                                                \
  do {                                                                                     \
    if (PHASE == PHASE_K) {                                                                \
      const float mk_ = (((kt_stage) % a.n_ftiles) == ftile) ? 1.f : 0.f;                  \
      _Pragma("unroll") for (int i = 0; i < CH_B; ++i) ee_rows[i] += mk_ * sumsq8(rb[i]);  \
    }                                                                                      \
  } while (0)

  // MFMA operand fragments, double-buffered across the 4 sub-steps of a k-step
  const int arow0 = wf * WF + (lane & 31);
  const int brow0 = wt * WT + (lane & 31);
  const int khalf = lane >> 5;
  bf16x8 fa[2][MF], fb[2][MT];
#define ENGRAM_LOAD_FRAGS(buf, la_, lb_, s_)                                               \
  do {                                                                                     \
    const int c_ = (s_) * 2 + khalf;                                                       \
    _Pragma("unroll") for (int i = 0; i < MF; ++i) {                                       \
      const int r_ = arow0 + i * 32;                                                       \
      fa[buf][i] = *reinterpret_cast<const bf16x8*>((la_) + r_ * BK + swz(r_, c_) * 8);    \
    }                                                                                      \
    _Pragma("unroll") for (int j = 0; j < MT; ++j) {                                       \
      const int r_ = brow0 + j * 32;                                                       \
      fb[buf][j] = *reinterpret_cast<const bf16x8*>((lb_) + r_ * BK + swz(r_, c_) * 8);    \
    }                                                                                      \
  } while (0)
#define ENGRAM_MFMAS(buf)                                                                  \
  do {                                                                                     \
    _Pragma("unroll") for (int i = 0; i < MF; ++i)                                         \
        _Pragma("unroll") for (int j = 0; j < MT; ++j)                                     \
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j],    \
                                                                 acc[i][j], 0, 0, 0);      \
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
  ENGRAM_EE(0);
  ENGRAM_STORE_STAGE(0);
  lds_barrier();
  ENGRAM_LOAD_FRAGS(0, smem, smem + STAGE_A, 0);

  // k-steps with a successor: MFMAs on LDS buffer kt & 1 while stage kt+1 loads into
  // registers; then stage kt+1 goes to the other buffer, last read in k-step kt-1
  // (finished before the previous barrier).  Scheduling barriers pin the order that
  // hides latency: global loads first, each sub-step's fragment reads a full sub-step
  // (16 MFMAs) ahead of their use, LDS writes last.
  for (int kt = 0; kt + 1 < nk; ++kt) {
    const uint16_t* la = smem + (kt & 1) * STAGE;
    const uint16_t* lb = la + STAGE_A;
    ENGRAM_LOAD_STAGE(kt + 1);
    __builtin_amdgcn_sched_barrier(0);
    ENGRAM_LOAD_FRAGS(1, la, lb, 1);
    ENGRAM_MFMAS(0);
    __builtin_amdgcn_sched_barrier(0);
    ENGRAM_LOAD_FRAGS(0, la, lb, 2);
    ENGRAM_MFMAS(1);
    __builtin_amdgcn_sched_barrier(0);
    ENGRAM_LOAD_FRAGS(1, la, lb, 3);
    ENGRAM_MFMAS(0);
    __builtin_amdgcn_sched_barrier(0);
    ENGRAM_MFMAS(1);
    __builtin_amdgcn_sched_barrier(0);
    ENGRAM_EE(kt + 1);
    ENGRAM_STORE_STAGE((kt + 1) & 1);
    lds_barrier();
    const uint16_t* na = smem + ((kt + 1) & 1) * STAGE;
    ENGRAM_LOAD_FRAGS(0, na, na + STAGE_A, 0);
  }
  // Last k-step.  The other stage buffer is free (last read in k-step nk-2): once this
  // step's fragment reads are issued, the half of the epilogue's h tile that lives
  // there starts loading straight into LDS, behind the remaining 32 MFMAs.
  const uint16_t* Ht0 = H + t0 * d_model;
  {
    const uint16_t* la = smem + ((nk - 1) & 1) * STAGE;
    const uint16_t* lb = la + STAGE_A;
    ENGRAM_LOAD_FRAGS(1, la, lb, 1);
    ENGRAM_MFMAS(0);
    __builtin_amdgcn_sched_barrier(0);
    ENGRAM_LOAD_FRAGS(0, la, lb, 2);
    ENGRAM_MFMAS(1);
    __builtin_amdgcn_sched_barrier(0);
    ENGRAM_LOAD_FRAGS(1, la, lb, 3);
    load_h_half(smem, Ht0, t0, n_tok, f0, d_model, nk & 1, wave, lane);
    ENGRAM_MFMAS(0);
    __builtin_amdgcn_sched_barrier(0);
    ENGRAM_MFMAS(1);
  }
#undef ENGRAM_LOAD_STAGE
#undef ENGRAM_STORE_STAGE
#undef ENGRAM_EE
#undef ENGRAM_LOAD_FRAGS
#undef ENGRAM_MFMAS
#undef ENGRAM_A_OFF
#undef ENGRAM_B_OFF

  // Everything below re-derives its indices from an opaque copy of the thread id, so
  // the compiler cannot compute epilogue addresses before the loop and keep them
  // live (in registers the main loop needs) across it.
  int etid = tid;
  asm volatile("" : "+v"(etid));
  const int elane = etid & 63, ewave = etid >> 6;
  const int ewf = ewave >> 1, ewt = ewave & 1;

  if (PHASE == PHASE_K) {
    // rows tid / ROW_CH + 32 i: the ROW_CH lanes of a row hold its partial sums
    float* ee_out = a.ee + ((int64_t)m * a.n_ftiles + ftile) * n_tok + t0;
#pragma unroll
    for (int i = 0; i < CH_B; ++i) {
      float v = ee_rows[i];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      const int r = etid / ROW_CH + 32 * i;
      if ((etid % ROW_CH) == 0 && t0 + r < n_tok) st_coherent(ee_out + r, v);
    }
  }

  // ---- the other half of the h tile, into the buffer the last k-step read
  __syncthreads();
  load_h_half(smem, Ht0, t0, n_tok, f0, d_model, (nk - 1) & 1, ewave, elane);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's direct-to-LDS loads have landed
  __syncthreads();

  // Lane (token column tl) holds, for MFMA tile (i, j) and pair gp, features
  // fl = wf*WF + i*32 + gp*16 + (lane>>5)*8 + 0..7 in acc[i][j][8*gp + 0..7].
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
            const u32x4 hv = *reinterpret_cast<const u32x4*>(smem + tl * BF + c * 8);
            const u32x4 gv = *reinterpret_cast<const u32x4*>(GQ + f0 + fl);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float h0 = bf16_lo(hv[q]), h1 = bf16_hi(hv[q]);
              dot += h0 * bf16_lo(gv[q]) * acc[i][j][gp * 8 + 2 * q];
              dot += h1 * bf16_hi(gv[q]) * acc[i][j][gp * 8 + 2 * q + 1];
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
      st_coherent(a.part_dot + o, s_red[0][0][etid] + s_red[1][0][etid]);
      st_coherent(a.part_hh + o, s_red[0][1][etid] + s_red[1][1][etid]);
    }
    // publish: __syncthreads() waits until every wave's partial stores have completed,
    // then the count goes up
    __syncthreads();
    if (etid == 0) __hip_atomic_fetch_add(done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
          u32x4* cell = reinterpret_cast<u32x4*>(smem + tl * BF + c * 8);
          const u32x4 hv = *cell;
          u32x4 ov;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            ov[q] = pack_bf16(bf16_lo(hv[q]) + alpha * acc[i][j][gp * 8 + 2 * q],
                              bf16_hi(hv[q]) + alpha * acc[i][j][gp * 8 + 2 * q + 1]);
          *cell = ov;
        }
      }
    }
    __syncthreads();
    uint16_t* Ot0 = (uint16_t*)a.out[m] + t0 * d_model;
#pragma unroll 8
    for (int i = 0; i < H_LOADS; ++i) {
      const int p = i * NTHR + etid;
      const int tl = p / H_CH;
      const int phys = p % H_CH;
      const int c = phys ^ (tl & 31);
      const int f = f0 + c * 8;
      if (t0 + tl < n_tok && f < d_model)
        *reinterpret_cast<u32x4*>(Ot0 + (uint32_t)tl * (uint32_t)d_model + f) =
            *reinterpret_cast<const u32x4*>(smem + p * 8);
    }
  }
}

__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gate_persistent_kernel(const GateArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM_ELEMS];  // stages, then h tile
  __shared__ float s_red[2][2][BT];  // [feature-wave][dot, hh][token]
  __shared__ float s_alpha[BT];
  __shared__ int s_tile;
  const int x = blockIdx.x % NQ;
  for (;;) {
    if (threadIdx.x == 0) s_tile = atomicAdd(a.counters + x, 1);
    __syncthreads();
    Tile t;
    const bool have = decode_tile(a, x, s_tile, t);
    __syncthreads();  // every thread has read s_tile before it is claimed again
    if (!have) break;
    gate_tile(a, t, smem, s_red, s_alpha);
    __syncthreads();  // LDS free for the next tile
  }
}

// One launch before the gate: W'[m][i][j] = bf16(W_K[m][i][j] * gk[m][j]) for every
// branch, and the tile queues / done counters cleared.
__global__ __launch_bounds__(256) void gate_prep_kernel(const GateArgs a, uint16_t* wk_scaled,
                                                        int64_t n8_per_branch, int n_counters) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_counters) a.counters[i] = 0;
  if (i >= n8_per_branch * a.n_branch) return;
  const int m = (int)(i / n8_per_branch);
  const int64_t k = i - m * n8_per_branch;
  const int j = (int)((k * 8) % a.d_mem);
  const u32x4 wv = reinterpret_cast<const u32x4*>(a.wk[m])[k];
  const u32x4 gv = *reinterpret_cast<const u32x4*>((const uint16_t*)a.gk[m] + j);
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = pack_bf16(bf16_lo(wv[q]) * bf16_lo(gv[q]), bf16_hi(wv[q]) * bf16_hi(gv[q]));
  reinterpret_cast<u32x4*>(wk_scaled)[i] = o;
}

struct ScratchLayout {
  size_t wk_bytes, part_bytes, counter_bytes, total;
  int n_counters;
};

ScratchLayout layout_for(const GateArgs& a) {
  ScratchLayout L;
  L.wk_bytes = ((size_t)a.n_branch * a.d_model * a.d_mem * 2 + 255) & ~(size_t)255;
  const size_t part_elems = (size_t)a.n_branch * a.n_ftiles * (size_t)a.n_tok;
  L.part_bytes = (part_elems * 4 + 255) & ~(size_t)255;
  L.n_counters = NQ + a.n_branch * a.n_ttiles;
  L.counter_bytes = ((size_t)L.n_counters * 4 + 255) & ~(size_t)255;
  L.total = L.wk_bytes + 3 * L.part_bytes + L.counter_bytes;
  return L;
}

int cu_count() {
  static int n[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (n[dev] == 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    n[dev] = c;
  }
  return n[dev];
}

}  // namespace

size_t gate_bf16_scratch_bytes(GateArgs& a) {
  a.n_ftiles = (a.d_model + BF - 1) / BF;
  a.n_ttiles = (int32_t)((a.n_tok + BT - 1) / BT);
  return layout_for(a).total;
}

// `a.part_dot` must point at the scratch block of gate_bf16_scratch_bytes(a) bytes;
// the other scratch pointers are carved from it here.
void launch_gate_bf16(const GateArgs& a_in, hipStream_t s) {
  GateArgs a = a_in;
  const ScratchLayout L = layout_for(a);
  char* base = (char*)a_in.part_dot;
  uint16_t* wk_scaled = (uint16_t*)base;
  a.part_dot = (float*)(base + L.wk_bytes);
  a.part_hh = (float*)(base + L.wk_bytes + L.part_bytes);
  a.ee = (float*)(base + L.wk_bytes + 2 * L.part_bytes);
  a.counters = (int32_t*)(base + L.wk_bytes + 3 * L.part_bytes);

  const int64_t n8 = (int64_t)a.d_model * a.d_mem / 8;
  const int64_t work = n8 * a.n_branch > L.n_counters ? n8 * a.n_branch : L.n_counters;
  hipLaunchKernelGGL(gate_prep_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, a,
                     wk_scaled, n8, L.n_counters);
  for (int m = 0; m < a.n_branch; ++m) a.wk[m] = wk_scaled + (size_t)m * a.d_model * a.d_mem;

  int grid = cu_count() / NQ * NQ;
  if (grid < NQ) grid = NQ;
  hipLaunchKernelGGL(gate_persistent_kernel, dim3((unsigned)grid), dim3(NTHR), 0, s, a);
}

}  // namespace engram
