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
// Main loop.  BK = 32 per k-step over a ring of four 32-KB LDS slots (weight rows
// and memory rows of one k-step each).  Operands move global -> LDS with direct
// loads (no registers), issued three k-steps ahead: three stages are in flight
// while the fourth is read, enough to cover the latency of L2 misses that a
// single register-staged stage could not.  The loads are issued from inline asm
// and waited for with explicit vmcnt counts, because the compiler would otherwise
// make every LDS read wait for all of them.  One LDS-only barrier per k-step both
// publishes the next stage and frees the slot just read.  The fragment registers
// are double-buffered so that a sub-step's MFMAs cover the next sub-step's LDS
// reads.  Slot rows are 64 B; the 16-B chunk index is XOR-swizzled by slot_key so
// the fragment reads (32 consecutive rows, one chunk) are free of bank conflicts.
//
// Epilogue.  The slot ring is reused for the h tile (256 tokens x 256 features,
// 128 KB): once no stage is left to load, each freed slot receives one quarter of
// it, behind the last k-steps' MFMAs; 16-byte chunks
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
constexpr int BK = 32;    // contraction depth per k-step
constexpr int NTHR = 256;
constexpr int WF = 128, WT = 128;           // per-wavefront tile
constexpr int MF = WF / 32, MT = WT / 32;   // MFMA tiles per wavefront
constexpr int NSLOT = 4;                    // LDS ring slots: 3 stages in flight + 1 being read
constexpr int SLOT_A_BYTES = BF * BK * 2;   // weight rows of a slot (64 B each)
constexpr int SLOT_BYTES = (BF + BT) * BK * 2;
constexpr int G_INSTR = SLOT_BYTES / 1024 / (NTHR / 64);  // 16-B-per-lane loads per wave per slot (8)
constexpr int H_CH = BF / 8;                // 16-B chunks per h row in the epilogue tile (32)
constexpr int H_LOADS = BT * H_CH / NTHR;   // 32 chunks per thread
constexpr int SMEM_ELEMS = (NSLOT * SLOT_BYTES / 2 > BT * BF) ? NSLOT * SLOT_BYTES / 2 : BT * BF;
static_assert(NSLOT * SLOT_BYTES == BT * BF * 2, "the h tile fills the slot ring exactly");
static_assert(NSLOT == 4 && G_INSTR == 8, "wait counts below assume 4 slots of 8 loads per wave");
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

// A slot row is 64 B (4 chunks of 16 B); logical chunk c of row r sits at physical
// chunk c ^ slot_key(r).  Eight consecutive rows at one logical chunk, and four
// consecutive rows at two neighbouring logical chunks, then cover distinct 16-B
// bank groups, so the fragment reads are conflict-free.
__device__ __forceinline__ int slot_key(int r) { return ((r >> 2) & 1) | (r & 2); }

typedef __attribute__((address_space(3))) void* lds_ptr;

// One 16-byte-per-lane direct global->LDS load: lane l's 16 bytes from `src` land at
// LDS byte address lds + 16 l (lds must be wave-uniform).  Issued from inline asm so
// that the compiler does not serialise later LDS reads behind it; completion is
// tracked by hand with wait_vm_lgkm0.  The compiler writes M0 (the LDS address
// operand); one wait state separates that write from the load that reads it.
__device__ __forceinline__ void dma16(const uint16_t* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// s_waitcnt vmcnt(N) lgkmcnt(0): at most N of this wave's vector-memory operations
// still in flight, and all its LDS operations done.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
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

  // ---- operand staging: a ring of NSLOT LDS slots, filled by direct global->LDS
  // loads issued DIST k-steps ahead.  Every wave issues exactly G_INSTR load
  // instructions per ring step ("group"): groups 0..NSLOT-1 in the prologue, group
  // kt + NSLOT right after the barrier that ends k-step kt, into the slot k-step kt
  // has just finished reading.  Group g is stage g while g < nk, else the h-tile
  // quarter that lands in slot g % NSLOT (the epilogue's h tile fills the whole ring).
  // So before the barrier that ends k-step kt, stage kt+1 has landed once at most
  // 2 G_INSTR of this wave's loads are still in flight (groups kt+2, kt+3).
  //
  // Waves 0-1 load weight rows 0-127 / 128-255, waves 2-3 memory rows; instruction i
  // of a wave fills rows (8 (wave & 1) + i) * 16 .. + 15 of its operand: lane l reads
  // row + l / 4, physical chunk l % 4 (logical chunk (l % 4) ^ key(row)).
  const int nk = d_mem / BK;
  const uint16_t* Et0 = E + t0 * d_mem;   // memory rows of this token tile
  const uint16_t* Ht0 = H + t0 * d_model;
  const int b_lim = (int)(n_tok - 1 - t0);  // last valid row of the token tile
  const bool wave_loads_a = (wave >> 1) == 0;
  const uint16_t* src_base = wave_loads_a ? W : Et0;
  // Row of instruction i: 16 i + (first row of instruction 0); both operands' rows
  // advance by 16 per instruction (the weight row permutation only touches bits 2-3),
  // and rows past the last valid one are clamped to it (their results are unused):
  // offset_i = min(src_off0 + i * src_step, src_lim).
  uint32_t src_off0, src_step, src_lim;
  {
    const int lrow = lane >> 2;
    const int lchunk = (lane & 3) ^ slot_key(lrow);  // slot_key only sees bits 1-2 of the row
    const int r0 = (wave & 1) * G_INSTR * 16 + lrow;
    const int row0 = wave_loads_a ? f0 + tile_row_feature(r0) : r0;
    const int last = wave_loads_a ? d_model - 1 : b_lim;
    src_off0 = (uint32_t)row0 * (uint32_t)d_mem + (uint32_t)(lchunk * 8);
    src_step = 16u * (uint32_t)d_mem;
    src_lim = (uint32_t)last * (uint32_t)d_mem + (uint32_t)(lchunk * 8);
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr)smem;
  const uint32_t wave_dst = lds0 + (uint32_t)((wave >> 1) * SLOT_A_BYTES + (wave & 1) * G_INSTR * 1024);

  // stage g (< nk) into slot g % NSLOT
#define ENGRAM_ISSUE_STAGE(g)                                                              \
  do {                                                                                     \
    const uint16_t* src_ = src_base + (g) * BK;                                            \
    const uint32_t dst_ = wave_dst + (uint32_t)(((g) % NSLOT) * SLOT_BYTES);               \
    _Pragma("unroll") for (int i = 0; i < G_INSTR; ++i)                                    \
        dma16(src_ + min(src_off0 + (uint32_t)i * src_step, src_lim), dst_ + i * 1024);    \
  } while (0)
  // h-tile quarter q (tokens 64 q .. 64 q + 63) into slot q, two token rows per
  // instruction; LDS chunk tl * 32 + phys holds logical chunk phys ^ (tl & 31) of
  // token tl.  Addresses come from an opaque copy of the lane id so that they are
  // not computed ahead and kept live through the main loop.
  auto issue_hq = [&](int q) {
    int hl = lane;
    asm volatile("" : "+v"(hl));
    const uint32_t slot_lds = lds0 + (uint32_t)(q * SLOT_BYTES);
#pragma unroll
    for (int i = 0; i < G_INSTR; ++i) {
      const int blk = wave * G_INSTR + i;
      const int tl = q * 64 + blk * 2 + (hl >> 5);
      const int c = (hl & 31) ^ (tl & 31);
      const int tr = tl < b_lim ? tl : b_lim;
      int f = f0 + c * 8;
      f = f < d_model ? f : 0;
      dma16(Ht0 + (uint32_t)tr * (uint32_t)d_model + f, slot_lds + (uint32_t)(blk * 1024));
    }
  };

  // MFMA operand fragments, double-buffered across the sub-steps.  Fragment row r of
  // a slot operand is 64 B; sub-step s of lane l reads logical chunk 2 s + l / 32.
  const int khalf = lane >> 5;
  const int arow0 = wf * WF + (lane & 31);
  const int brow0 = wt * WT + (lane & 31);
  uint32_t fr_a[2], fr_b[2];  // byte offsets inside a slot, per sub-step
#pragma unroll
  for (int ss = 0; ss < 2; ++ss) {
    fr_a[ss] = (uint32_t)(arow0 * (BK * 2) + (((ss * 2 + khalf) ^ slot_key(arow0)) * 16));
    fr_b[ss] = (uint32_t)(SLOT_A_BYTES + brow0 * (BK * 2) + (((ss * 2 + khalf) ^ slot_key(brow0)) * 16));
  }
  bf16x8 fa[2][MF], fb[2][MT];
#define ENGRAM_LOAD_FRAGS(buf, slot_base_, ss_)                                            \
  do {                                                                                     \
    const char* sb_ = (const char*)smem + (slot_base_);                                    \
    _Pragma("unroll") for (int i = 0; i < MF; ++i)                                         \
        fa[buf][i] = *reinterpret_cast<const bf16x8*>(sb_ + fr_a[ss_] + i * 32 * BK * 2);  \
    _Pragma("unroll") for (int j = 0; j < MT; ++j)                                         \
        fb[buf][j] = *reinterpret_cast<const bf16x8*>(sb_ + fr_b[ss_] + j * 32 * BK * 2);  \
  } while (0)
#define ENGRAM_MFMAS(buf)                                                                  \
  do {                                                                                     \
    _Pragma("unroll") for (int i = 0; i < MF; ++i)                                         \
        _Pragma("unroll") for (int j = 0; j < MT; ++j)                                     \
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j],    \
                                                                 acc[i][j], 0, 0, 0);      \
  } while (0)
  // Sum of e^2 over the k-steps kt with kt % n_ftiles == ftile, from the memory
  // fragments: waves with wf == 0 see every token row of the tile (lanes l and l+32
  // hold the two halves of a sub-step's 16 columns).
  float ee_acc[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) ee_acc[j] = 0.f;
  const bool ee_wave = PHASE == PHASE_K && wf == 0;
#define ENGRAM_EE(buf)                                                                     \
  do {                                                                                     \
    _Pragma("unroll") for (int j = 0; j < MT; ++j)                                         \
        ee_acc[j] += sumsq8(__builtin_bit_cast(u32x4, fb[buf][j]));                        \
  } while (0)

  floatx16 acc[MF][MT];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  for (int g = 0; g < NSLOT; ++g) {
    if (g < nk) ENGRAM_ISSUE_STAGE(g);
    else issue_hq(g);
  }
  wait_vm_lgkm0<3 * G_INSTR>();
  lds_barrier();
  // k-step 0: both sub-steps' fragments, sub-step 0's MFMAs
  ENGRAM_LOAD_FRAGS(0, 0, 0);
  ENGRAM_LOAD_FRAGS(1, 0, 1);
  ENGRAM_MFMAS(0);
  bool ee_prev = ee_wave && (0 % a.n_ftiles) == ftile;
  if (ee_prev) ENGRAM_EE(0);
  wait_vm_lgkm0<2 * G_INSTR>();
  lds_barrier();
  if (NSLOT < nk) ENGRAM_ISSUE_STAGE(NSLOT);
  else issue_hq(0);

  // k-step kt: sub-step 1 of k-step kt-1 (fragments already in registers) covers the
  // latency of this step's first fragment reads; then sub-step 0 of kt.  The barrier
  // at the end publishes stage kt+1 and frees slot kt % NSLOT for group kt + NSLOT:
  // a stage while one is left, else the h-tile quarter of that slot.
#define ENGRAM_KSTEP(kt)                                                                   \
  do {                                                                                     \
    const uint32_t slot_ = (uint32_t)(((kt) % NSLOT) * SLOT_BYTES);                        \
    ENGRAM_LOAD_FRAGS(0, slot_, 0);                                                        \
    __builtin_amdgcn_sched_barrier(0);                                                     \
    ENGRAM_MFMAS(1);                                                                       \
    __builtin_amdgcn_sched_barrier(0);                                                     \
    if (ee_prev) ENGRAM_EE(1);                                                             \
    ENGRAM_LOAD_FRAGS(1, slot_, 1);                                                        \
    __builtin_amdgcn_sched_barrier(0);                                                     \
    ENGRAM_MFMAS(0);                                                                       \
    __builtin_amdgcn_sched_barrier(0);                                                     \
    ee_prev = ee_wave && ((kt) % a.n_ftiles) == ftile;                                     \
    if (ee_prev) ENGRAM_EE(0);                                                             \
    wait_vm_lgkm0<2 * G_INSTR>();                                                          \
    lds_barrier();                                                                         \
  } while (0)
  int kt = 1;
  for (; kt + NSLOT < nk; ++kt) {
    ENGRAM_KSTEP(kt);
    ENGRAM_ISSUE_STAGE(kt + NSLOT);
  }
  for (; kt < nk; ++kt) {
    ENGRAM_KSTEP(kt);
    issue_hq(kt % NSLOT);
  }
#undef ENGRAM_KSTEP
#undef ENGRAM_ISSUE_STAGE
  ENGRAM_MFMAS(1);
  if (ee_prev) ENGRAM_EE(1);
#undef ENGRAM_EE
#undef ENGRAM_LOAD_FRAGS
#undef ENGRAM_MFMAS

  // Everything below re-derives its indices from an opaque copy of the thread id, so
  // the compiler cannot compute epilogue addresses before the loop and keep them
  // live (in registers the main loop needs) across it.
  int etid = tid;
  asm volatile("" : "+v"(etid));
  const int elane = etid & 63, ewave = etid >> 6;
  const int ewf = ewave >> 1, ewt = ewave & 1;

  if (ee_wave) {
    // lanes l and l + 32 of a wf == 0 wave hold the two halves of token row
    // ewt * WT + j * 32 + l % 32
    float* ee_out = a.ee + ((int64_t)m * a.n_ftiles + ftile) * n_tok + t0;
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const float v = ee_acc[j] + __shfl_xor(ee_acc[j], 32, 64);
      const int r = ewt * WT + j * 32 + (elane & 31);
      if (elane < 32 && t0 + r < n_tok) st_coherent(ee_out + r, v);
    }
  }

  // ---- the h tile: its four quarters were loaded into the ring as it drained
  wait_vm_lgkm0<0>();
  lds_barrier();

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
