// gate_bf16.hip -- context-aware gating on the gfx950 matrix cores (bf16 operands, or E4M3
// codes for the FP8 form; fp32 accumulation).
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
//   K tile: acc = W_K' e^T for (feature tile, token tile), with
//           W_K'[f][c] = gq[f] W_K[f][c] gk[c] (both RMSNorm gains folded in,
//           prepared once per call by gate_prep_kernel); the epilogue reduces
//           sum_f h[t,f] acc[f,t] and sum_f h[t,f]^2 over the tile's features into
//           per-(feature tile, token) partials; the main loop also sums e^2 over
//           one slice of the memory row (k-steps with kt % n_ftiles == ftile), so
//           every tile does 1/n_ftiles of it.  The last K tile of a (branch, token
//           tile) to finish turns the partials into alpha (fixed-order sums:
//           bit-reproducible) and publishes it;
//   V tile: computes acc = W_V e^T, waits until alpha of its (branch, token tile)
//           is published (usually long before) and writes out = h + alpha acc.
// Since q . k = (sum_f h_f gq_f k~_f) / (rms(h) rms(e)) with k~ = W_K diag(gk) e,
// the RMSNorm scales are applied to the reduced scalar, never to a tensor.
// The same sum is also sum_c e_c u_c with u = W_K'^T h: with d_mem < d_model and
// enough tokens the K tiles take that memory-major form (TK below: tiles of 256 memory
// dimensions contracting over d_model, h streamed, the memory rows in the epilogue),
// fewer and longer tiles for the same FLOPs.
//
// Scheduling.  One persistent launch of one workgroup per CU.  Workgroup b
// serves work queue b % 8 (the XCD it is dispatched to), which holds the token
// tiles T with T % 8 == b % 8: first all their K tiles, then all their V tiles.
// Within a phase the tiles come in blocks of 4 token tiles x 8 (branch, feature
// tile) pairs, so the 32 CUs of an XCD working on one block at a time share each
// memory tile 8 ways and each weight panel 4 ways in the XCD's L2 (rather than
// one memory tile 32 ways and 32 distinct weight panels, which the L2 cannot hold:
// 44 % less traffic to the fabric and a 4 % faster gate on the large workload).
// A workgroup claims the next tile of its queue with an
// atomic increment (the next one already when the current tile's epilogue
// starts, so the claim's latency is hidden); before its epilogue a V tile spins
// until the done-counter of its K tiles is full.  Those K tiles sit earlier in the
// same queue, so they were claimed before by running workgroups that never wait:
// the spin always ends.  The single queue per XCD removes the partial last round of
// a two-launch design (640 + 640 tiles on 256 CUs become 1280 = 5 x 256) and keeps
// a token tile's memory rows in one XCD's L2.
//
// Tiling.  256 features x 256 tokens per tile, four wavefronts in 2 x 2, each
// owning 128 x 128 outputs = 4 x 4 MFMA 32x32 tiles (256 fp32 accumulators per
// lane).  Features are the MFMA rows, so all 16 accumulators of a lane in one
// MFMA tile belong to ONE token; weight rows are loaded in a permuted order
// (bits 2 and 3 of the row index swapped inside each 32-row tile) so that a
// lane's accumulator groups 0-1 and 2-3 each cover 8 consecutive features:
// every epilogue access is a 16-byte vector.
//
// Main loop.  BK = 64 per k-step over a ring of five 32-KB LDS slots, each holding
// one operand of one k-step (256 weight rows or 256 memory rows of 128 B).
// Operands move global -> LDS with direct loads (no registers); the refill of the
// two slots a k-step frees is spread through that k-step's MFMA stream, so three
// slots are in flight while two are read, enough to cover the latency of L2 misses.
// The loads are issued from inline asm and waited for with explicit vmcnt counts,
// because the compiler would otherwise make every LDS read wait for all of them.
// One LDS-only barrier per k-step both publishes the next stage and frees the slots
// just read.  The fragment reads are spread one per two MFMAs in the order the
// MFMAs consume them.  The 16-B chunk index of a row is XOR-swizzled by row_key so
// the fragment reads (32 consecutive rows, one chunk) are free of bank conflicts.
//
// Epilogue.  The slot ring is reused for the h tile (256 tokens x 256 features,
// 128 KB): once no stage is left to load, each freed slot receives one quarter of
// it, behind the last k-steps' MFMAs; 16-byte chunks
// are swizzled by (token & 31) so that 32 lanes reading 32 tokens hit distinct
// banks.  A V tile writes out into the same LDS tile and then streams it to
// HBM with coalesced 16-byte stores.
//
// Variants.  The persistent kernel is instantiated per option (gate_tile lists them):
// the gated-value output, the paper's projected key norm, one W_V shared by all
// branches, and FP8 operands (E4M3 codes, 32x32x64 MFMA, 128 k-values per ring row).
// Each is its own instantiation so that the plain gate keeps its register allocation.
#include <atomic>

#include "engram_internal.h"

namespace engram {

// Wavefronts of V tiles whose bounded wait for their gates ran out (they wrote NaN),
// per device, since the library was loaded or the count was last reset.
__device__ int32_t g_gate_wait_timeouts;

// Tile timeline (a diagnostic build only, libengram_timeline.so, compiled with
// ENGRAM_GATE_TIMELINE): thread 0 of each workgroup stamps s_memrealtime (100 MHz) at the
// phase boundaries of each of its first TL_TILES tiles, in g_timeline[workgroup][tile][point]:
//   0 loop top (claim published)  1 tile decoded  2 first operands landed  3 main loop done
//   4 h tile landed  5 V gates in LDS  6 epilogue done  7 after the end-of-tile barrier
//   K tiles: 8 dot pass done  9 partial stores issued  10 stores acknowledged  11 count raised
//   V tiles: 12 output tile in LDS  13 output streamed
//   15: the tile (phase | branch << 1 | feature tile << 4 | token tile << 16)
// In the normal build ENGRAM_STAMP expands to nothing.
#ifdef ENGRAM_GATE_TIMELINE
constexpr int TL_WGS = 256, TL_TILES = 512, TL_POINTS = 16;
__device__ uint64_t g_timeline[TL_WGS * TL_TILES * TL_POINTS];
#define ENGRAM_TL_SLOT(k) g_timeline[((int64_t)blockIdx.x * TL_TILES + tl_n) * TL_POINTS + (k)]
#define ENGRAM_STAMP(k)                                                        \
  do {                                                                         \
    if (threadIdx.x == 0 && blockIdx.x < TL_WGS && tl_n < TL_TILES)            \
      ENGRAM_TL_SLOT(k) = __builtin_amdgcn_s_memrealtime();                    \
  } while (0)
#define ENGRAM_STAMP_TILE(t)                                                   \
  do {                                                                         \
    if (threadIdx.x == 0 && blockIdx.x < TL_WGS && tl_n < TL_TILES)            \
      ENGRAM_TL_SLOT(15) = (uint64_t)(t).phase | ((uint64_t)(t).m << 1) |      \
                           ((uint64_t)(t).ftile << 4) | ((uint64_t)(t).ttile << 16); \
  } while (0)
#else
#define ENGRAM_STAMP(k) \
  do {                  \
  } while (0)
#define ENGRAM_STAMP_TILE(t) \
  do {                       \
  } while (0)
#endif

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16-B chunk (native: stays in registers)
typedef int v8i __attribute__((ext_vector_type(8)));          // FP8 MFMA operand: 32 E4M3 codes
typedef int v4i_t __attribute__((ext_vector_type(4)));

constexpr int BF = 256;   // features per tile
constexpr int BT = 256;   // tokens per tile
constexpr int BK = 64;    // contraction depth per k-step
constexpr int NTHR = 256;
constexpr int WF = 128, WT = 128;           // per-wavefront tile
constexpr int MF = WF / 32, MT = WT / 32;   // MFMA tiles per wavefront
constexpr int NSLOT = 5;                    // LDS ring slots
constexpr int SLOT_BYTES = 256 * BK * 2;    // one operand of one k-step: 256 rows x 128 B
constexpr int G_INSTR = SLOT_BYTES / 1024 / (NTHR / 64);  // 16-B-per-lane loads per wave per slot (8)
constexpr int H_CH = BF / 8;                // 16-B chunks per h row in the epilogue tile (32)
constexpr int H_LOADS = BT * H_CH / NTHR;   // 32 chunks per thread
constexpr int SMEM_BYTES = NSLOT * SLOT_BYTES;  // 160 KB: the whole LDS of a CU
static_assert(4 * SLOT_BYTES == BT * BF * 2, "the h tile is four slots");
static_assert(G_INSTR == 8 && BF == 256 && BT == 256, "load and wait counts below assume these");
constexpr int NQ = 8;                       // work queues (one per XCD)
constexpr int SPIN_LIMIT = 1 << 18;         // polls (each one L2 round trip plus s_sleep 1: 0.1-0.5 s) before a V tile gives up
constexpr int FORCED_SPIN_LIMIT = 64;       // polls of a wait made unsatisfiable on purpose (test hook)

enum { PHASE_K = 0, PHASE_V = 1 };

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  // round-to-nearest-even conversion (v_cvt_pk_bf16_f32 on gfx950).  Kept as two
  // scalar conversions: the two-lane vector form saves a few instructions but changes
  // the persistent kernel's register allocation (more spills, 2 % slower measured).
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// A slot row is 128 B (8 chunks of 16 B); logical chunk c of row r sits at
// physical chunk c ^ row_key(r).  The fragment reads (32 consecutive rows at one
// logical chunk) then touch every bank group once per 8 rows: conflict-free.
__device__ __forceinline__ int row_key(int r) { return (r & 7) ^ ((r >> 3) & 1); }

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
// at the device coherence point without flushing or invalidating whole caches.
// Publishing is ordered by hand: every wave waits for its own stores with
// s_waitcnt vmcnt(0) (on gfx9 a store leaves the vmcnt count only once the memory
// side has acknowledged it, and an agent-scope store is acknowledged at the device
// coherence point), then the workgroup barrier, and only then one thread
// increments the done counter.  __syncthreads() alone is not enough: on gfx950 its
// workgroup-scope fence waits for LDS operations but not for global stores.  A
// reader issues its loads only after the load of the count that showed them
// complete has returned (its branch depends on the value).  Full acquire/release at
// device scope would write back and invalidate the XCD's L2 on every tile,
// evicting the operand tiles the other CUs are streaming.
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Tile {
  int phase, m, ttile, ftile;
};

// Tile q of queue x; false once the queue is exhausted.  SHAREDV (all branches share
// W_V): one V tile per (token tile, feature tile) serves every branch, so the V phase
// has n_branch times fewer tiles; its tiles carry m = 0.
constexpr int TT_GROUP = 4;   // token tiles per group
constexpr int CB = 8;         // (branch, feature tile) combinations per block
// the gathering gate (its memory tiles are random table rows): the same, its own sizes
constexpr int TT_GROUP_G = 4;
constexpr int CB_G = 8;
// the V phase behind memory-major key tiles: 8 token tiles x 4 pairs (measured 0.5-1.4 % faster
// than 4 x 8 there on the large and multi workloads; 4 x 8 stays the faster one behind
// feature-major key tiles)
constexpr int TT_GROUP_TKV = 8;
constexpr int CB_TKV = 4;

// Tile r of a phase whose tiles are the n_tt token tiles of a queue x `per` combinations
// (branch, feature tile), ordered so that 32 consecutive tiles cover TTG token tiles x CBN
// combinations (each memory tile shared by CBN tiles, each weight panel by TTG).
template <int TTG, int CBN>
__device__ __forceinline__ void blocked(int r, int n_tt, int per, int& tt, int& combo) {
  const int g = r / (TTG * per);
  const int ntt = min(TTG, n_tt - g * TTG);
  const int rg = r - g * TTG * per;
  const int cb = rg / (ntt * CBN);
  const int cbs = min(CBN, per - cb * CBN);
  const int rb = rg - cb * ntt * CBN;
  tt = g * TTG + rb / cbs;
  combo = cb * CBN + rb % cbs;
}

// The same order with run-time block sizes (memory-major K tiles).
__device__ __forceinline__ void blocked_rt(int r, int n_tt, int per, int ttg, int cbn, int& tt, int& combo) {
  const int g = r / (ttg * per);
  const int ntt = min(ttg, n_tt - g * ttg);
  const int rg = r - g * ttg * per;
  const int cb = rg / (ntt * cbn);
  const int cbs = min(cbn, per - cb * cbn);
  const int rb = rg - cb * ntt * cbn;
  tt = g * ttg + rb / cbs;
  combo = cb * cbn + rb % cbs;
}

template <bool SHAREDV, bool GATHER, bool TK>
__device__ __forceinline__ bool decode_tile(const GateArgs& a, int x, int q, Tile& t) {
  const int n_tt = a.n_ttiles > x ? (a.n_ttiles - x + NQ - 1) / NQ : 0;  // token tiles of queue x
  if constexpr (TK) {
    // n_ktiles K tiles per (branch, token tile), n_ftiles V tiles
    const int per_k_tt = a.n_branch * a.n_ktiles;
    const int per_v_tt = SHAREDV ? a.n_ftiles : a.n_branch * a.n_ftiles;
    const int per_k = n_tt * per_k_tt;
    const int per_v = n_tt * per_v_tt;
    if (q >= per_k + per_v) return false;
    t.phase = q >= per_k ? PHASE_V : PHASE_K;
    const int r = q - (t.phase == PHASE_V ? per_k : 0);
    const int per = t.phase == PHASE_V ? per_v_tt : per_k_tt;
    int tl, combo;
    // K tiles stream h, which is per branch: a block is one branch's n_ktiles tiles of 32
    // token tiles, taken token tile by token tile, so an XCD's 32 CUs run about
    // 32 / n_ktiles token tiles' key tiles at a time (each h tile shared n_ktiles ways, each
    // weight panel that many token tiles' ways) and stay on one branch's weight panels for
    // 32 token tiles (measured 0.5 % faster than switching branch every 32 / n_ktiles)
    if (t.phase == PHASE_K) blocked_rt(r, n_tt, per, 32, a.n_ktiles, tl, combo);
    else blocked<TT_GROUP_TKV, CB_TKV>(r, n_tt, per, tl, combo);
    const int nt = t.phase == PHASE_V ? a.n_ftiles : a.n_ktiles;  // output tiles per branch
    t.m = combo / nt;
    t.ftile = combo - t.m * nt;
    t.ttile = tl * NQ + x;
    return true;
  }
  const int per_tt = a.n_branch * a.n_ftiles;
  const int per_k = n_tt * per_tt;
  const int per_v = SHAREDV ? n_tt * a.n_ftiles : per_k;
  if (q >= per_k + per_v) return false;
  t.phase = q >= per_k ? PHASE_V : PHASE_K;
  const int r = q - (t.phase == PHASE_V ? per_k : 0);
  const int per = (SHAREDV && t.phase == PHASE_V) ? a.n_ftiles : per_tt;
  int tl, combo;
  if constexpr (GATHER) blocked<TT_GROUP_G, CB_G>(r, n_tt, per, tl, combo);
  else blocked<TT_GROUP, CB>(r, n_tt, per, tl, combo);
  t.m = combo / a.n_ftiles;
  t.ftile = combo - t.m * a.n_ftiles;
  t.ttile = tl * NQ + x;
  return true;
}

// One K or V tile.  A single main loop serves both phases (one copy of the
// loop keeps register allocation simple); only the epilogues differ.  Two options,
// each its own instantiation so that the plain gate keeps its register allocation:
//   VALUES  the V epilogue also writes the gated values alpha * v where a branch asks
//           for them;
//   KEYP    the paper's key placement, k = RMSNorm_gk(W_K e) with gk over d_model: the
//           K tiles run on the raw W_K, their epilogue weights h_f by gq_f gk_f (from
//           LDS) and also reduces sum_f k_f^2, which takes the place of the e^2 partial;
//   SHAREDV every branch uses the same W_V (section 2.4, Eq. (6)): a V tile computes
//           W_V e once, waits for the gates of all branches, and runs one epilogue per
//           branch, loading that branch's h tile into the ring between them;
//   F8      the projections in FP8 (section 2.4): both operands are E4M3 codes with one
//           fp32 scale per row (per token for e, per feature for the weights), prepared
//           by the quantization kernels.  A 128-byte ring row then holds 128 k-values,
//           and each MFMA (32x32x64 E4M3) takes one 64-value half; the feature scales
//           weight the epilogues from LDS, the token scale joins the reduced scalars;
//   GATHER  (bf16) the memory rows are not read from a memory-vector array: each lane
//           hashes its token's n-grams and its direct loads read the table rows in
//           place (gs, a GatherSrc; NoGather otherwise);
//   TK      (bf16, memory-side key norm) memory-major K tiles.  The logit's dot product
//           is also sum_c u_c e_c with u = W_K'^T h: a K tile computes u for 256 memory
//           dimensions c x 256 tokens, contracting over d_model (a.wk[m] then holds
//           W_K'^T, [d_mem][d_model]), with h as the streamed token operand and the
//           memory rows as the epilogue tile.  Its epilogue reduces sum_c e_c u_c and
//           sum_c e_c^2, its main loop sums h^2 over one slice of d_model.  Same FLOPs,
//           but ceil(d_mem / 256) K tiles per (branch, token tile) instead of
//           ceil(d_model / 256), each d_model / 64 k-steps long: the fixed cost of a
//           tile's edges (first operands, epilogue, publishing) is paid fewer times.
//           The V tiles are the feature-major ones of the other instantiations.
struct NoGather {};

template <bool VALUES, bool KEYP, bool SHAREDV, bool F8, bool GATHER, bool TK, class GS>
__device__ __forceinline__ void gate_tile(const GateArgs& a, const GS& gs, const Tile& tile, char* smem, int x,
                                          int& next_claim, int tl_n) {
  ENGRAM_STAMP(1);
  ENGRAM_STAMP_TILE(tile);
  static_assert(!(GATHER && F8), "the gathering gate is bf16");
  static_assert(!TK || (!KEYP && !F8 && !GATHER), "memory-major K tiles: bf16, memory-side key norm, no gather");
  // TK: the tile's fields are made wave-uniform (scalar registers) here.  The tile number
  // reaches every lane through LDS, so the compiler would otherwise keep the values derived
  // from it in vector registers; with the phase-dependent row lengths and bases of the TK
  // main loop that spilled address registers whose reloads the compiler then waited for
  // inside the k-step loop (s_waitcnt vmcnt(0), which also drains the operand ring).
  const int PHASE = TK ? __builtin_amdgcn_readfirstlane(tile.phase) : tile.phase;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wf = wave >> 1, wt = wave & 1;
  const int m = TK ? __builtin_amdgcn_readfirstlane(tile.m) : tile.m;
  const int ftile = TK ? __builtin_amdgcn_readfirstlane(tile.ftile) : tile.ftile;
  const int f0 = ftile * BF;
  const int64_t t0 = (int64_t)(TK ? __builtin_amdgcn_readfirstlane(tile.ttile) : tile.ttile) * BT;
  const int64_t n_tok = a.n_tok;
  const int d_mem = a.d_mem, d_model = a.d_model;
  int32_t* done = a.counters + NQ + m * a.n_ttiles + tile.ttile;

  // phase K reads the gain-folded copy of W_K (a.wk points at it here), or KEYP W_K itself
  const uint16_t* W = (const uint16_t*)(PHASE == PHASE_K ? a.wk[m] : a.wv[m]);
  const uint16_t* E = (const uint16_t*)a.mem;
  const uint16_t* H = (const uint16_t*)a.h[m];
  // TK K tiles swap the roles of the memory rows and h: Lrow is the length of the
  // streamed rows (the contraction depth), Dout the extent of the tile's output rows and
  // the row length of its epilogue tile
  const bool tk = TK && PHASE == PHASE_K;
  const int Lrow = tk ? d_model : d_mem;
  const int Dout = tk ? d_mem : d_model;
  const int nkt = tk ? a.n_ktiles : a.n_ftiles;  // tiles sharing this tile's token rows and phase

  // ---- V tiles need the gates of their (branch, token tile), published by its last K
  // tile (done count n_ktiles + 1), only in the epilogue.  Each wave looks at the count
  // once here: if the gates are out, it fetches its tokens' gates now and the loads
  // complete behind the main loop; if not, it runs the main loop anyway and waits after
  // it (with few tiles in flight, as in a decode step, V tiles then overlap K tiles).
  float alpha = 0.f;  // V tiles: the gate of token t0 + tid (to LDS once the ring drains)
  bool gates_ready = true;  // wave-uniform
  if (PHASE == PHASE_V) {
    int seen = 1;
    if (lane == 0) {
      for (int mb = SHAREDV ? 0 : m; mb < (SHAREDV ? a.n_branch : m + 1); ++mb)
        seen &= __hip_atomic_load(a.counters + NQ + mb * a.n_ttiles + tile.ttile, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT) >= (TK ? a.n_ktiles : a.n_ftiles) + 1 + a.wait_extra;
    }
    gates_ready = __builtin_amdgcn_readfirstlane(seen) != 0;
    // issued only after lane 0's count came back (the branch depends on it)
    if (gates_ready && t0 + tid < n_tok) alpha = ld_coherent(a.alpha + (int64_t)m * n_tok + t0 + tid);
  }
  float kg = 0.f;  // KEYP K tiles: gq * gk of feature f0 + tid (to LDS in the epilogue)
  if (KEYP && PHASE == PHASE_K && f0 + tid < d_model) kg = a.kgain[(int64_t)m * d_model + f0 + tid];
  // F8: the weight scale of feature f0 + tid (K or V weights; 0 past d_model), and for V
  // tiles the token scale of token t0 + tid; both to LDS in the epilogue
  float fs = 0.f, ts = 0.f;
  if constexpr (F8) {
    if (f0 + tid < d_model) fs = (PHASE == PHASE_K ? a.sk[m] : a.sv[m])[f0 + tid];
    if (PHASE == PHASE_V && t0 + tid < n_tok) ts = a.se[t0 + tid];
  }

  // ---- operand stream.  Chunk c of the tile's stream lands in LDS slot c % NSLOT:
  // chunks 2 kt and 2 kt + 1 are the weight rows and the memory rows of k-step kt
  // (256 rows x 128 B each), chunks 2 nk .. 2 nk + 3 the four quarters of the
  // epilogue's h tile.  Chunks 0-4 are issued up front.  The barrier that ends
  // k-step kt - 1 frees its two slots, and during k-step kt chunks 2 kt + 3 and
  // 2 kt + 4 are issued into them, spread through the MFMA stream (one load after
  // every four MFMAs) so that a full load queue delays a few MFMAs instead of
  // stalling all of them at once.  Every chunk is G_INSTR direct global->LDS loads
  // per wave, so at the end of k-step kt, when chunks 2 kt + 2 and 2 kt + 3 must
  // have landed, at most the G_INSTR loads of chunk 2 kt + 4 may be in flight.
  //
  // Instruction i of wave w fills rows 64 w + 8 i .. + 7 of a chunk: lane l reads
  // row 64 w + 8 i + l / 8 at physical chunk l % 8 (logical (l % 8) ^ row_key).
  const int nk = Lrow / (F8 ? 2 * BK : BK);  // k-steps of 128 bytes per row
  // the streamed token rows of this token tile (memory rows; TK K tiles: h rows) and the
  // rows of its epilogue tile (h; TK K tiles: memory rows)
  const uint16_t* Et0 = tk ? H + t0 * d_model : E + t0 * d_mem;
  const uint16_t* Ht0 = tk ? E + t0 * d_mem : H + t0 * d_model;
  const int b_lim = (int)(n_tok - 1 - t0);  // last valid row of the token tile
  uint32_t off_a[G_INSTR], off_b[G_INSTR];
#pragma unroll
  for (int i = 0; i < G_INSTR; ++i) {
    const int r = wave * 64 + i * 8 + (lane >> 3);
    const int cl = (lane & 7) ^ row_key(r);
    // weight rows are permuted (tile_row_feature); rows past the end are clamped to
    // the last valid one (their results are unused)
    off_a[i] = (uint32_t)min(f0 + tile_row_feature(r), Dout - 1) * (uint32_t)Lrow + cl * (F8 ? 16 : 8);
    off_b[i] = (uint32_t)min(r, b_lim) * (uint32_t)Lrow + cl * (F8 ? 16 : 8);
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr)smem;
  const uint32_t wave_dst = lds0 + (uint32_t)(wave * G_INSTR * 1024);

  // ---- GATHER: the memory rows of k-step k are chunks 8 k .. 8 k + 7 of each token's
  // concatenated row: chunk gO + c of its row in table gT, or past that row's end chunk
  // gO + c - cpr of its row in table gT + 1 (gO = 8 k - gT * cpr < cpr, and cpr >= 8, so
  // no k-step reaches a third table).  Lane L of wave w keeps token w * 64 + L's
  // canonical ids and its row numbers in tables gT and gT + 1, hashing the next table's
  // as gT advances; instruction i of the wave loads tokens w * 64 + 8 i + L / 8, whose
  // row numbers it takes from lane 8 i + L / 8 (ds_bpermute).  Memory rows are issued in
  // k-step order, each k-step's once, and each k-step's preparation is three steps:
  //   gather_prep   the permutes (LDS operations only);
  //   gather_fetch  the scalar loads of the tables' bases and, if the state will enter a
  //                 new table, that table's hash constants; waited for at once (an
  //                 outstanding scalar load would turn every later LDS wait into a full
  //                 one), so the main loop calls it just before the end-of-k-step wait,
  //                 which waits for everything anyway;
  //   gather_step   the state moves on, hashing with the fetched constants.
  // In the main loop the permutes for the next iteration go out once this iteration's
  // memory loads are issued, and each load's address is formed right before it, in the
  // shadow of an MFMA.
  struct GHash {
    uint64_t m0, m1, m2, m3, bar;
    uint32_t rows;
    int order;
    bool adv;
  };
  uint32_t gpv0[G_INSTR], gpv1[G_INSTR];  // row numbers of the next memory chunk
  int gpo = 0;                            // ... its offset in its first table
  const char* gpb[2] = {nullptr, nullptr};  // ... the bases of its two tables
  GHash gph{};                            // ... and what the state needs after it
  uint32_t gx0 = 0, gx1 = 0, gx2 = 0, gx3 = 0, gi0 = 0, gi1 = 0;
  int gT = 0, gO = 0, gcpr = 8, gnt = 1;
  auto hash_row = [&](const GHash& c) -> uint32_t {
    uint64_t hv = (uint64_t)gx0 * c.m0;
    if (c.order > 1) hv ^= (uint64_t)gx1 * c.m1;
    if (c.order > 2) hv ^= (uint64_t)gx2 * c.m2;
    if (c.order > 3) hv ^= (uint64_t)gx3 * c.m3;
    return mod_barrett(hv, c.rows, c.bar);
  };
  auto hash_consts = [&](int tb) -> GHash {
    GHash c{};
    if constexpr (GATHER) {
      c.m0 = gs.mult[tb][0];
      c.m1 = gs.mult[tb][1];
      c.m2 = gs.mult[tb][2];
      c.m3 = gs.mult[tb][3];
      c.bar = gs.barrett[tb];
      c.rows = gs.rows[tb];
      c.order = gs.order[tb];
    }
    return c;
  };
  auto gather_prep = [&](uint32_t (&v0)[G_INSTR], uint32_t (&v1)[G_INSTR], int& o) {
    if constexpr (GATHER) {
#pragma unroll
      for (int i = 0; i < G_INSTR; ++i)
        v0[i] = (uint32_t)__builtin_amdgcn_ds_bpermute((i * 8 + (lane >> 3)) * 4, (int)gi0);
      // table gT + 1 only if some chunk of the k-step lies in it (otherwise no lane selects v1)
      if (gO + 7 >= gcpr) {
#pragma unroll
        for (int i = 0; i < G_INSTR; ++i)
          v1[i] = (uint32_t)__builtin_amdgcn_ds_bpermute((i * 8 + (lane >> 3)) * 4, (int)gi1);
      }
      o = gO;
    }
  };
  // (the fetched values are made opaque wave-uniform values: a per-lane choice between
  // the two bases must select values, not become a per-lane load)
  auto gather_fetch = [&](const char* (&base)[2], GHash& c) {
    if constexpr (GATHER) {
      base[0] = gs.tab[gT];
      base[1] = gs.tab[gT + 1 < gnt ? gT + 1 : gT];
      c.adv = gO + 8 >= gcpr;
      if (c.adv && gT + 2 < gnt) {
        const GHash h = hash_consts(gT + 2);
        c.m0 = h.m0;
        c.m1 = h.m1;
        c.m2 = h.m2;
        c.m3 = h.m3;
        c.bar = h.bar;
        c.rows = h.rows;
        c.order = h.order;
      }
      asm volatile("" : "+s"(base[0]), "+s"(base[1]), "+s"(c.m0), "+s"(c.m1), "+s"(c.m2), "+s"(c.m3),
                   "+s"(c.bar), "+s"(c.rows), "+s"(c.order));
    }
  };
  auto gather_step = [&](const GHash& c) {
    if constexpr (GATHER) {
      gO += 8;
      if (c.adv) {
        gO -= gcpr;
        ++gT;
        gi0 = gi1;
        gi1 = gT + 1 < gnt ? hash_row(c) : 0u;
      }
    }
  };
  // the address of load instruction i's 16-byte chunk (lane l: logical chunk
  // (l % 8) ^ row_key(row), as for the memory-vector array)
  auto gather_addr = [&](int i, const uint32_t (&v0)[G_INSTR], const uint32_t (&v1)[G_INSTR], int o,
                         const char* const (&base)[2]) -> const uint16_t* {
    const int r = wave * 64 + i * 8 + (lane >> 3);
    const int q = o + ((lane & 7) ^ row_key(r));
    const bool next = q >= gcpr;
    const uint32_t z = next ? v1[i] : v0[i];
    const char* bp = next ? base[1] : base[0];
    return (const uint16_t*)(bp + (uint64_t)z * ((uint32_t)gcpr * 16u) + (uint32_t)(next ? q - gcpr : q) * 16u);
  };
  if constexpr (GATHER) {
    gcpr = gs.cpr;
    gnt = gs.n_tables;
    asm volatile("" : "+s"(gcpr), "+s"(gnt));
    const int4 v = gs.ids[t0 + min(wave * 64 + lane, b_lim)];
    gx0 = (uint32_t)v.x;
    gx1 = (uint32_t)v.y;
    gx2 = (uint32_t)v.z;
    gx3 = (uint32_t)v.w;
    gi0 = hash_row(hash_consts(0));
    gi1 = gnt > 1 ? hash_row(hash_consts(1)) : 0u;
  }
#define ENGRAM_ISSUE(base_, off_, kt_, slot_)                                              \
  do {                                                                                     \
    const uint16_t* src_ = (base_) + (kt_) * BK;                                           \
    const uint32_t dst_ = wave_dst + (uint32_t)((slot_) * SLOT_BYTES);                     \
    _Pragma("unroll") for (int i = 0; i < G_INSTR; ++i)                                    \
        dma16(src_ + off_[i], dst_ + i * 1024);                                            \
  } while (0)
  // h-tile quarter q (tokens 64 q .. 64 q + 63) into slot `slot`, two token rows per
  // instruction; byte (tl % 64) * 512 + 16 phys of the quarter holds logical chunk
  // phys ^ (tl & 31) of token tl.  Addresses come from an opaque copy of the lane id
  // so that they are not computed ahead and kept live through the main loop.
  auto issue_hq = [&](int q, int slot) {
    int hl = lane;
    asm volatile("" : "+v"(hl));
    const uint32_t dst = lds0 + (uint32_t)(slot * SLOT_BYTES);
#pragma unroll
    for (int i = 0; i < G_INSTR; ++i) {
      const int blk = wave * G_INSTR + i;
      const int tl = q * 64 + blk * 2 + (hl >> 5);
      const int c = (hl & 31) ^ (tl & 31);
      const int tr = tl < b_lim ? tl : b_lim;
      int f = f0 + c * 8;
      f = f < Dout ? f : 0;
      dma16(Ht0 + (uint32_t)tr * (uint32_t)Dout + f, dst + (uint32_t)(blk * 1024));
    }
  };
  // FP8: the operands are byte arrays (offsets above are in bytes)
  const uint8_t* W8 = (const uint8_t*)W;
  const uint8_t* Et8 = (const uint8_t*)E + t0 * d_mem;
#define ENGRAM_ISSUE8(base_, off_, kt_, slot_)                                             \
  do {                                                                                     \
    const uint8_t* src_ = (base_) + (kt_) * (2 * BK);                                      \
    const uint32_t dst_ = wave_dst + (uint32_t)((slot_) * SLOT_BYTES);                     \
    _Pragma("unroll") for (int i = 0; i < G_INSTR; ++i)                                    \
        dma16((const uint16_t*)(src_ + off_[i]), dst_ + i * 1024);                        \
  } while (0)
  // any chunk (the prologue and the last k-steps)
  auto issue_chunk = [&](int c) {
    const int slot = c % NSLOT;
    if (c < 2 * nk) {
      if constexpr (F8) {
        if (c & 1) ENGRAM_ISSUE8(Et8, off_b, c >> 1, slot);
        else ENGRAM_ISSUE8(W8, off_a, c >> 1, slot);
      } else if constexpr (GATHER) {
        if (c & 1) {
          uint32_t v0[G_INSTR], v1[G_INSTR];
          int o;
          const char* base[2];
          GHash c{};
          gather_prep(v0, v1, o);
          gather_fetch(base, c);
          gather_step(c);
          const uint32_t dst = wave_dst + (uint32_t)(slot * SLOT_BYTES);
#pragma unroll
          for (int i = 0; i < G_INSTR; ++i) dma16(gather_addr(i, v0, v1, o, base), dst + i * 1024);
        } else {
          ENGRAM_ISSUE(W, off_a, c >> 1, slot);
        }
      } else {
        if (c & 1) ENGRAM_ISSUE(Et0, off_b, c >> 1, slot);
        else ENGRAM_ISSUE(W, off_a, c >> 1, slot);
      }
    } else {
      issue_hq(c - 2 * nk, slot);
    }
  };

  // MFMA operand fragments, double-buffered across the 4 sub-steps of a k-step;
  // sub-step s of lane l reads logical chunk 2 s + l / 32 of rows (l % 32) + 32 i.
  const int khalf = lane >> 5;
  const int arow0 = wf * WF + (lane & 31);
  const int brow0 = wt * WT + (lane & 31);
  uint32_t fr_a[4], fr_b[4];
#pragma unroll
  for (int ss = 0; ss < 4; ++ss) {
    fr_a[ss] = (uint32_t)(arow0 * (BK * 2) + (((ss * 2 + khalf) ^ row_key(arow0)) * 16));
    fr_b[ss] = (uint32_t)(brow0 * (BK * 2) + (((ss * 2 + khalf) ^ row_key(brow0)) * 16));
  }
  bf16x8 fa[2][MF], fb[2][MT];
  // Reads are issued in the order the MFMAs consume them (row i = 0 of the weight
  // fragments with all memory fragments, then the other weight rows), so the first
  // MFMAs wait for two reads, not five.
#define ENGRAM_LOAD_FRAGS(buf, sa_, sb_, ss_)                                              \
  do {                                                                                     \
    const char* pa_ = smem + (sa_) + fr_a[ss_];                                            \
    const char* pb_ = smem + (sb_) + fr_b[ss_];                                            \
    fa[buf][0] = *reinterpret_cast<const bf16x8*>(pa_);                                    \
    _Pragma("unroll") for (int j = 0; j < MT; ++j)                                         \
        fb[buf][j] = *reinterpret_cast<const bf16x8*>(pb_ + j * 32 * BK * 2);              \
    _Pragma("unroll") for (int i = 1; i < MF; ++i)                                         \
        fa[buf][i] = *reinterpret_cast<const bf16x8*>(pa_ + i * 32 * BK * 2);              \
  } while (0)
#define ENGRAM_MFMAS(buf)                                                                  \
  do {                                                                                     \
    _Pragma("unroll") for (int i = 0; i < MF; ++i)                                         \
        _Pragma("unroll") for (int j = 0; j < MT; ++j)                                     \
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j],    \
                                                                 acc[i][j], 0, 0, 0);      \
  } while (0)
  // One fragment read (n = 0..7, in the order the MFMAs consume them) of sub-step ss_.
#define ENGRAM_READ1(buf, sa_, sb_, ss_, n)                                                \
  do {                                                                                     \
    if ((n) == 0)                                                                          \
      fa[buf][0] = *reinterpret_cast<const bf16x8*>(smem + (sa_) + fr_a[ss_]);             \
    else if ((n) <= MT)                                                                    \
      fb[buf][(n) - 1] = *reinterpret_cast<const bf16x8*>(smem + (sb_) + fr_b[ss_] +       \
                                                          ((n) - 1) * 32 * BK * 2);        \
    else                                                                                   \
      fa[buf][(n) - MT] = *reinterpret_cast<const bf16x8*>(smem + (sa_) + fr_a[ss_] +      \
                                                           ((n) - MT) * 32 * BK * 2);      \
  } while (0)
  // The 16 MFMAs of fragment buffer bm, with the next sub-step's eight fragment reads
  // (sub-step rs into buffer br) spread one after every second MFMA, and, when
  // dma_, load instructions q0 .. q0 + 3 of an operand chunk one after every fourth.
  // Spreading the reads (rather than issuing all eight at once) measured 12 % faster:
  // bursts of fragment reads and direct-to-LDS writes contend for the LDS.
#define ENGRAM_GROUP(bm, br, rs, sa_, sb_, dma_, gat_, base_, off_, kt_, slot_, q0)        \
  do {                                                                                     \
    const uint16_t* src_ = (base_) + (kt_) * BK;                                           \
    const uint32_t dst_ = wave_dst + (uint32_t)((slot_) * SLOT_BYTES);                     \
    _Pragma("unroll") for (int k_ = 0; k_ < MF * MT; ++k_) {                               \
      acc[k_ / MT][k_ % MT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                     \
          fa[bm][k_ / MT], fb[bm][k_ % MT], acc[k_ / MT][k_ % MT], 0, 0, 0);               \
      __builtin_amdgcn_sched_barrier(0);                                                   \
      if ((k_ % 2) == 0) {                                                                 \
        ENGRAM_READ1(br, sa_, sb_, rs, k_ / 2);                                            \
        __builtin_amdgcn_sched_barrier(0);                                                 \
      }                                                                                    \
      if ((dma_) && (k_ % MT) == MT - 1) {                                                 \
        if (GATHER && (gat_))                                                              \
          dma16(gather_addr((q0) + k_ / MT, gpv0, gpv1, gpo, gpb),                         \
                dst_ + ((q0) + k_ / MT) * 1024);                                           \
        else                                                                               \
          dma16(src_ + off_[(q0) + k_ / MT], dst_ + ((q0) + k_ / MT) * 1024);              \
        __builtin_amdgcn_sched_barrier(0);                                                 \
      }                                                                                    \
    }                                                                                      \
  } while (0)
  // Sum of e^2 (TK K tiles: h^2) over the k-steps kt with kt % nkt == ftile, from the
  // token-row fragments: waves with wf == 0 see every token row of the tile (lanes l and l+32
  // hold the two halves of a sub-step's 16 columns).
  float ee_acc[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) ee_acc[j] = 0.f;
  const bool ee_wave = !KEYP && !F8 && PHASE == PHASE_K && wf == 0;
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

  if constexpr (!F8) {
  for (int c = 0; c < NSLOT; ++c) issue_chunk(c);
  wait_vm_lgkm0<3 * G_INSTR>();
  lds_barrier();
  ENGRAM_STAMP(2);
  // k-step 0, sub-steps 0-2 (sub-step 3's MFMAs open k-step 1); no slot is free yet
  bool ee_now = ee_wave && ftile == 0;
  ENGRAM_LOAD_FRAGS(0, 0, SLOT_BYTES, 0);
  ENGRAM_LOAD_FRAGS(1, 0, SLOT_BYTES, 1);
  ENGRAM_MFMAS(0);
  if (ee_now) ENGRAM_EE(0);
  ENGRAM_LOAD_FRAGS(0, 0, SLOT_BYTES, 2);
  ENGRAM_MFMAS(1);
  if (ee_now) ENGRAM_EE(1);
  if (GATHER && 3 < nk) gather_prep(gpv0, gpv1, gpo);  // k-step 2, the main loop's first
  ENGRAM_LOAD_FRAGS(1, 0, SLOT_BYTES, 3);
  ENGRAM_MFMAS(0);
  if (ee_now) ENGRAM_EE(0);
  if (GATHER && 3 < nk) gather_fetch(gpb, gph);
  wait_vm_lgkm0<G_INSTR>();
  lds_barrier();
  if (GATHER && 3 < nk) gather_step(gph);

  // k-step kt: the MFMAs of sub-step 3 of k-step kt-1 (fragments in registers) cover
  // this step's first fragment reads, each later sub-step's MFMAs cover the next one's
  // reads.  A load of the operand stream follows every fourth MFMA when dma_; the
  // barrier at the end publishes k-step kt+1 and frees k-step kt's slots.
#define ENGRAM_KSTEP(kt, dma_, b0_, o0_, k0_, s0_, b1_, o1_, k1_, s1_)                     \
  do {                                                                                     \
    const int sa_ = ((2 * (kt)) % NSLOT) * SLOT_BYTES;                                     \
    const int sb_ = ((2 * (kt) + 1) % NSLOT) * SLOT_BYTES;                                 \
    __builtin_amdgcn_sched_barrier(0);                                                     \
    ENGRAM_GROUP(1, 0, 0, sa_, sb_, dma_, true, b0_, o0_, k0_, s0_, 0);                    \
    if (ee_now) ENGRAM_EE(1);                                                              \
    ee_now = ee_wave && ((kt) % nkt) == ftile;                                             \
    ENGRAM_GROUP(0, 1, 1, sa_, sb_, dma_, true, b0_, o0_, k0_, s0_, 4);                    \
    if (ee_now) ENGRAM_EE(0);                                                              \
    /* GATHER: the next iteration's row numbers; the wait at the end covers them */      \
    if (GATHER && (kt) + 3 < nk) gather_prep(gpv0, gpv1, gpo);                             \
    ENGRAM_GROUP(1, 0, 2, sa_, sb_, dma_, false, b1_, o1_, k1_, s1_, 0);                   \
    if (ee_now) ENGRAM_EE(1);                                                              \
    ENGRAM_GROUP(0, 1, 3, sa_, sb_, dma_, false, b1_, o1_, k1_, s1_, 4);                   \
    if (ee_now) ENGRAM_EE(0);                                                              \
    __builtin_amdgcn_sched_barrier(0);                                                     \
    if (GATHER && (kt) + 3 < nk) gather_fetch(gpb, gph);                                   \
    wait_vm_lgkm0<G_INSTR>();                                                              \
    lds_barrier();                                                                         \
    if (GATHER && (kt) + 3 < nk) gather_step(gph);                                         \
  } while (0)
  int kt = 1;
  // chunks 2 kt + 3 (memory rows of k-step kt + 1) and 2 kt + 4 (weight rows of
  // k-step kt + 2) into the slots k-step kt - 1 freed
  for (; kt + 2 < nk; ++kt)
    ENGRAM_KSTEP(kt, true, Et0, off_b, kt + 1, (2 * kt + 3) % NSLOT, W, off_a, kt + 2,
                 (2 * kt + 4) % NSLOT);
  // The last k-steps: the stream ends with the h-tile quarters, issued as a burst;
  // each sub-step's fragments are read in one burst too (measured faster here than
  // spreading them, behind the burst of h-tile loads).
  for (; kt < nk; ++kt) {
    issue_chunk(2 * kt + 3);
    issue_chunk(2 * kt + 4);
    const int sa = ((2 * kt) % NSLOT) * SLOT_BYTES;
    const int sb = ((2 * kt + 1) % NSLOT) * SLOT_BYTES;
    ENGRAM_LOAD_FRAGS(0, sa, sb, 0);
    __builtin_amdgcn_sched_barrier(0);
    ENGRAM_MFMAS(1);
    __builtin_amdgcn_sched_barrier(0);
    if (ee_now) ENGRAM_EE(1);
    ee_now = ee_wave && (kt % nkt) == ftile;
    ENGRAM_LOAD_FRAGS(1, sa, sb, 1);
    __builtin_amdgcn_sched_barrier(0);
    ENGRAM_MFMAS(0);
    __builtin_amdgcn_sched_barrier(0);
    if (ee_now) ENGRAM_EE(0);
    ENGRAM_LOAD_FRAGS(0, sa, sb, 2);
    __builtin_amdgcn_sched_barrier(0);
    ENGRAM_MFMAS(1);
    __builtin_amdgcn_sched_barrier(0);
    if (ee_now) ENGRAM_EE(1);
    ENGRAM_LOAD_FRAGS(1, sa, sb, 3);
    __builtin_amdgcn_sched_barrier(0);
    ENGRAM_MFMAS(0);
    __builtin_amdgcn_sched_barrier(0);
    if (ee_now) ENGRAM_EE(0);
    wait_vm_lgkm0<G_INSTR>();
    lds_barrier();
  }
  issue_chunk(2 * nk + 3);
  ENGRAM_MFMAS(1);
  if (ee_now) ENGRAM_EE(1);
  } else {
    // ---- FP8 main loop.  The same ring and chunk numbering; a 128-byte k-step is two
    // halves of 64 k-values, and the fragment of a half is the two 16-byte chunks that
    // the bf16 loop reads for two consecutive sub-steps (logical chunks 4 p + khalf and
    // 4 p + 2 + khalf), for both operands alike.  A weight fragment register is reloaded
    // as soon as its last MFMA has issued (row i after MFMA (i, MT-1)); the memory
    // fragments, each used by every row, are double-buffered (half p in set p) and read
    // one after every second MFMA from the start of the other half:
    //   half 0 of k-step kt, reading half 1 of kt and loading chunk 2 kt + 4 (weight
    //   rows of kt + 2) into the slot k-step kt - 1's memory rows left;
    //   wait + barrier: k-step kt + 1 has landed, k-step kt's slots are free;
    //   half 1 of kt, reading half 0 of kt + 1 and loading chunk 2 kt + 5 (memory rows
    //   of kt + 2) into kt's weight slot.
    // The loads go one after every second MFMA, as in the bf16 loop; in the last two
    // k-steps, where the chunks are h-tile quarters, as a burst before the MFMAs.  Only
    // chunk 2 kt + 4 may be in flight at the barrier of kt.  No branch may enter the
    // MFMA sequences (the compiler would move the MFMAs past it): the last k-step reads
    // fragments it does not use.
    v8i fa8[MF], fb8[2][MT];  // B fragments double-buffered: half 0 in set 0, half 1 in set 1
    auto frag8 = [&](int base, uint32_t o0, uint32_t o1) -> v8i {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(smem + base + o0);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(smem + base + o1);
      return __builtin_shufflevector(__builtin_bit_cast(v4i_t, lo), __builtin_bit_cast(v4i_t, hi), 0, 1, 2, 3, 4,
                                     5, 6, 7);
    };
#define ENGRAM_F8_A(sa_, p_, i_) fa8[i_] = frag8((sa_) + (i_) * 32 * 2 * BK, fr_a[2 * (p_)], fr_a[2 * (p_) + 1])
#define ENGRAM_F8_B(sb_, p_, j_) fb8[p_][j_] = frag8((sb_) + (j_) * 32 * 2 * BK, fr_b[2 * (p_)], fr_b[2 * (p_) + 1])
#define ENGRAM_F8_MFMA(p_, i_, j_)                                                         \
  acc[i_][j_] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa8[i_], fb8[p_][j_], acc[i_][j_], 0, 0, 0, 127, 0, 127)
#define ENGRAM_F8_KSTEP(spread_)                                                           \
  do {                                                                                     \
    const int sa = ((2 * kt) % NSLOT) * SLOT_BYTES;                                        \
    const int sb = ((2 * kt + 1) % NSLOT) * SLOT_BYTES;                                    \
    if (!(spread_)) issue_chunk(2 * kt + 4);                                               \
    const uint8_t* srcW = W8 + (kt + 2) * (2 * BK);                                        \
    const uint32_t dstW = wave_dst + (uint32_t)(((2 * kt + 4) % NSLOT) * SLOT_BYTES);      \
    __builtin_amdgcn_sched_barrier(0);                                                     \
    _Pragma("unroll") for (int k = 0; k < MF * MT; ++k) {                                  \
      ENGRAM_F8_MFMA(0, k / MT, k % MT);                                                   \
      __builtin_amdgcn_sched_barrier(0);                                                   \
      if ((k & 1) == 0 && k < 2 * MT) ENGRAM_F8_B(sb, 1, k >> 1);                          \
      if (k % MT == MT - 1) ENGRAM_F8_A(sa, 1, k / MT);                                    \
      if ((spread_) && (k & 1)) dma16((const uint16_t*)(srcW + off_a[k >> 1]), dstW + (k >> 1) * 1024); \
      __builtin_amdgcn_sched_barrier(0);                                                   \
    }                                                                                      \
    wait_vm_lgkm0<G_INSTR>();                                                              \
    lds_barrier();                                                                         \
    if (!(spread_)) issue_chunk(2 * kt + 5);                                               \
    const int sa2 = ((2 * kt + 2) % NSLOT) * SLOT_BYTES;                                   \
    const int sb2 = ((2 * kt + 3) % NSLOT) * SLOT_BYTES;                                   \
    const uint8_t* srcE = Et8 + (kt + 2) * (2 * BK);                                       \
    const uint32_t dstE = wave_dst + (uint32_t)sa;                                         \
    __builtin_amdgcn_sched_barrier(0);                                                     \
    _Pragma("unroll") for (int k = 0; k < MF * MT; ++k) {                                  \
      ENGRAM_F8_MFMA(1, k / MT, k % MT);                                                   \
      __builtin_amdgcn_sched_barrier(0);                                                   \
      if ((k & 1) == 0 && k < 2 * MT) ENGRAM_F8_B(sb2, 0, k >> 1);                         \
      if (k % MT == MT - 1) ENGRAM_F8_A(sa2, 0, k / MT);                                   \
      if ((spread_) && (k & 1)) dma16((const uint16_t*)(srcE + off_b[k >> 1]), dstE + (k >> 1) * 1024); \
      __builtin_amdgcn_sched_barrier(0);                                                   \
    }                                                                                      \
  } while (0)
    // chunks 0-3 (k-steps 0 and 1) up front; k-step 0 waits for its own two
    for (int c = 0; c < 4; ++c) issue_chunk(c);
    wait_vm_lgkm0<2 * G_INSTR>();
    lds_barrier();
    ENGRAM_STAMP(2);
#pragma unroll
    for (int j = 0; j < MT; ++j) ENGRAM_F8_B(SLOT_BYTES, 0, j);
#pragma unroll
    for (int i = 0; i < MF; ++i) ENGRAM_F8_A(0, 0, i);
    int kt = 0;
    // chunks 2 kt + 4 and 2 kt + 5 are both operand rows while kt + 3 <= nk
    for (; kt + 3 <= nk; ++kt) ENGRAM_F8_KSTEP(true);
    for (; kt < nk; ++kt) ENGRAM_F8_KSTEP(false);
#undef ENGRAM_F8_KSTEP
#undef ENGRAM_F8_A
#undef ENGRAM_F8_B
#undef ENGRAM_F8_MFMA
  }
#undef ENGRAM_KSTEP
#undef ENGRAM_GROUP
#undef ENGRAM_READ1
#undef ENGRAM_ISSUE
#undef ENGRAM_ISSUE8
#undef ENGRAM_EE
#undef ENGRAM_LOAD_FRAGS
#undef ENGRAM_MFMAS

  // Nothing of the epilogue may be scheduled into the last k-steps (measured: 8 %
  // slower when the compiler is free to interleave them).
  __builtin_amdgcn_sched_barrier(0);
  ENGRAM_STAMP(3);

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

  // ---- the h tile: quarter q is chunk 2 nk + q, in slot (2 nk + q) % NSLOT; the
  // fifth slot, (2 nk + 4) % NSLOT, holds the epilogue's cross-wave scratch
  wait_vm_lgkm0<0>();
  lds_barrier();
  ENGRAM_STAMP(4);
  // claim this workgroup's next tile now; the atomic's latency hides behind the epilogue
  if (tid == 0) next_claim = atomicAdd(a.counters + x, 1);
  // byte offset of h-tile quarter q (a runtime q must not index a local array: that
  // would live in scratch memory and cost a memory round trip per access)
  const int q0slot = (2 * nk) % NSLOT;
#define ENGRAM_QSLOT(q) ((q0slot + (q) >= NSLOT ? q0slot + (q) - NSLOT : q0slot + (q)) * SLOT_BYTES)
  char* scratch = smem + ((2 * nk + 4) % NSLOT) * SLOT_BYTES;
  float (*s_red)[2][BT] = reinterpret_cast<float (*)[2][BT]>(scratch);  // [feature-wave][dot, hh][token]
  float* s_alpha = reinterpret_cast<float*>(scratch + 4 * BT * sizeof(float));
  // LDS byte offset of logical 16-B chunk c of token tl in the h tile
#define ENGRAM_HOFF(tl, c) (ENGRAM_QSLOT((tl) >> 6) + ((tl) & 63) * (BF * 2) + (((c) ^ ((tl) & 31)) * 16))
  int* s_flag = reinterpret_cast<int*>(scratch + 5 * BT * sizeof(float));
  float (*s_kk)[BT] = reinterpret_cast<float (*)[BT]>(scratch + 6 * BT * sizeof(float));  // KEYP
  float* s_g = reinterpret_cast<float*>(scratch + 8 * BT * sizeof(float));               // KEYP, [BF]
  float* s_fs = reinterpret_cast<float*>(scratch + 8 * BT * sizeof(float) + BF * sizeof(float));  // F8, [BF]
  bool gave_up = false;  // wave-uniform: this wave's bounded wait for the gates ran out
  if (PHASE == PHASE_V) {
    if (!gates_ready) {
      // the wait deferred from the tile's start: lane 0 polls the done count(s), bounded
      // by a.spin_limit polls, and the wave's gate loads follow once it has seen them.
      // A wave that gives up counts itself in g_gate_wait_timeouts and takes NaN for
      // its gates, so its outputs are NaN rather than silently wrong.
      int out_of_polls = 0;
      if (elane == 0) {
        int spin = 0;
        for (int mb = SHAREDV ? 0 : m; mb < (SHAREDV ? a.n_branch : m + 1) && !out_of_polls; ++mb) {
          const int32_t* dn = a.counters + NQ + mb * a.n_ttiles + tile.ttile;
          while (__hip_atomic_load(dn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (TK ? a.n_ktiles : a.n_ftiles) + 1 + a.wait_extra) {
            if (++spin >= a.spin_limit) {
              out_of_polls = 1;
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
        }
        if (out_of_polls)
          __hip_atomic_fetch_add(&g_gate_wait_timeouts, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      gave_up = __builtin_amdgcn_readfirstlane(out_of_polls) != 0;
      if (gave_up) alpha = __builtin_nanf("");
      else if (t0 + etid < n_tok) alpha = ld_coherent(a.alpha + (int64_t)m * n_tok + t0 + etid);
    }
    if constexpr (F8) s_alpha[etid] = alpha * ts;  // the token scale rides on the gate
    else s_alpha[etid] = alpha;
    lds_barrier();
  }
  ENGRAM_STAMP(5);
  if (KEYP && PHASE == PHASE_K) {
    s_g[etid] = kg;
    lds_barrier();
  }

  // Lane (token column tl) holds, for MFMA tile (i, j) and pair gp, features
  // fl = wf*WF + i*32 + gp*16 + (lane>>5)*8 + 0..7 in acc[i][j][8*gp + 0..7].
  const int hsel = (elane >> 5) * 8;
  // F8: acc holds W e over each feature's weight scale.  The epilogues multiply each
  // accumulator by its feature's scale (from LDS) as they read it (FOLD; ENGRAM_WS: the
  // eight scales of features fl .. fl + 7), which gives the values the bf16 epilogues take
  // (k_f or v_f over the token scale), rounded the same way, without writing every scaled
  // accumulator back first.  With a shared W_V the V epilogue runs once per branch, so
  // there the accumulators are scaled once up front instead (fewer spills measured).  The
  // bf16 instantiations keep their own copies of those loops.
  constexpr bool FOLD = F8 && !SHAREDV;
  if constexpr (F8) {
    s_fs[etid] = fs;
    lds_barrier();
  }
  if constexpr (F8 && !FOLD) {
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        const int fl = ewf * WF + i * 32 + gp * 16 + hsel;
        const float4 g0 = *reinterpret_cast<const float4*>(s_fs + fl);
        const float4 g1 = *reinterpret_cast<const float4*>(s_fs + fl + 4);
        const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
        for (int j = 0; j < MT; ++j)
#pragma unroll
          for (int r = 0; r < 8; ++r) acc[i][j][gp * 8 + r] *= g[r];
      }
  }
#define ENGRAM_WS(fl_, ws_)                                                                 \
  const float4 ws_##_lo = *reinterpret_cast<const float4*>(s_fs + (fl_));                   \
  const float4 ws_##_hi = *reinterpret_cast<const float4*>(s_fs + (fl_) + 4);               \
  const float ws_[8] = {ws_##_lo.x, ws_##_lo.y, ws_##_lo.z, ws_##_lo.w,                     \
                        ws_##_hi.x, ws_##_hi.y, ws_##_hi.z, ws_##_hi.w}
  if (PHASE == PHASE_K) {
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int tl = ewt * WT + j * 32 + (elane & 31);
      // all eight cells first (no LDS writes in between, so the reads issue back to
      // back); rows past Dout (a ragged last tile) count as zero
      u32x4 hv[MF][2];
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          const int fl = ewf * WF + i * 32 + gp * 16 + hsel;
          hv[i][gp] = *reinterpret_cast<const u32x4*>(smem + ENGRAM_HOFF(tl, fl >> 3));
          if (f0 + fl >= Dout) hv[i][gp] = (u32x4){0u, 0u, 0u, 0u};
        }
      if constexpr (!KEYP) {
        float dot = 0.f, hh = 0.f, dot2 = 0.f, hh2 = 0.f;  // two chains each
        if constexpr (FOLD) {
#pragma unroll
          for (int i = 0; i < MF; ++i) {
#pragma unroll
            for (int gp = 0; gp < 2; ++gp) {
              ENGRAM_WS(ewf * WF + i * 32 + gp * 16 + hsel, ws);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float h0 = bf16_lo(hv[i][gp][q]), h1 = bf16_hi(hv[i][gp][q]);
                dot += h0 * (acc[i][j][gp * 8 + 2 * q] * ws[2 * q]);
                dot2 += h1 * (acc[i][j][gp * 8 + 2 * q + 1] * ws[2 * q + 1]);
                hh += h0 * h0;
                hh2 += h1 * h1;
              }
            }
          }
        } else {
#pragma unroll
        for (int i = 0; i < MF; ++i) {
#pragma unroll
          for (int gp = 0; gp < 2; ++gp) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float h0 = bf16_lo(hv[i][gp][q]), h1 = bf16_hi(hv[i][gp][q]);
              dot += h0 * acc[i][j][gp * 8 + 2 * q];
              dot2 += h1 * acc[i][j][gp * 8 + 2 * q + 1];
              hh += h0 * h0;
              hh2 += h1 * h1;
            }
          }
        }
        }
        dot += dot2;
        hh += hh2;
        dot += __shfl_xor(dot, 32, 64);
        hh += __shfl_xor(hh, 32, 64);
        if (elane < 32) {
          s_red[ewf][0][tl] = dot;
          s_red[ewf][1][tl] = hh;
        }
      } else {
        // q_f k_f with the gains from LDS; k_f^2 only over features that exist
        float dot = 0.f, hh = 0.f, kk = 0.f, dot2 = 0.f, hh2 = 0.f, kk2 = 0.f;
#pragma unroll
        for (int i = 0; i < MF; ++i) {
#pragma unroll
          for (int gp = 0; gp < 2; ++gp) {
            const int fl = ewf * WF + i * 32 + gp * 16 + hsel;
            const float4 g0 = *reinterpret_cast<const float4*>(s_g + fl);
            const float4 g1 = *reinterpret_cast<const float4*>(s_g + fl + 4);
            const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
            const float vm = f0 + fl < d_model ? 1.f : 0.f;
            float ws[8] = {};
            if constexpr (FOLD) {
              ENGRAM_WS(fl, wf8);
#pragma unroll
              for (int r = 0; r < 8; ++r) ws[r] = wf8[r];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float h0 = bf16_lo(hv[i][gp][q]), h1 = bf16_hi(hv[i][gp][q]);
              float a0 = acc[i][j][gp * 8 + 2 * q], a1 = acc[i][j][gp * 8 + 2 * q + 1];
              if constexpr (FOLD) {
                a0 *= ws[2 * q];
                a1 *= ws[2 * q + 1];
              }
              dot += h0 * g[2 * q] * a0;
              dot2 += h1 * g[2 * q + 1] * a1;
              hh += h0 * h0;
              hh2 += h1 * h1;
              kk += vm * a0 * a0;
              kk2 += vm * a1 * a1;
            }
          }
        }
        dot += dot2;
        hh += hh2;
        kk += kk2;
        dot += __shfl_xor(dot, 32, 64);
        hh += __shfl_xor(hh, 32, 64);
        kk += __shfl_xor(kk, 32, 64);
        if (elane < 32) {
          s_red[ewf][0][tl] = dot;
          s_red[ewf][1][tl] = hh;
          s_kk[ewf][tl] = kk;
        }
      }
    }
    ENGRAM_STAMP(8);
    __syncthreads();
    const int64_t t = t0 + etid;
    if (t < n_tok) {
      const int64_t o = ((int64_t)m * a.n_ftiles + ftile) * n_tok + t;
      st_coherent(a.part_dot + o, s_red[0][0][etid] + s_red[1][0][etid]);
      st_coherent(a.part_hh + o, s_red[0][1][etid] + s_red[1][1][etid]);
      if (KEYP) st_coherent(a.ee + o, s_kk[0][etid] + s_kk[1][etid]);
    }
    // publish: every wave waits for its own partial stores, then the barrier, then the
    // count goes up
    ENGRAM_STAMP(9);
    wait_vm_lgkm0<0>();
    __syncthreads();
    ENGRAM_STAMP(10);
    if (etid == 0) *s_flag = __hip_atomic_fetch_add(done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    lds_barrier();
    ENGRAM_STAMP(11);
    if (*s_flag == nkt - 1) {
      // The last K tile of this (branch, token tile): every other one stored its
      // partials before its increment, so all are in L2.  Turn them into gates
      // (fixed-order sums: bit-reproducible), publish, and count once more.
      const int64_t t = t0 + etid;
      if (t < n_tok) {
        const int nf = nkt;  // partials of this branch's K tiles (stride n_ftiles per branch)
        const int64_t base = (int64_t)m * a.n_ftiles * n_tok + t;
        float dot = 0.f, hh = 0.f, ee = 0.f;
        for (int j0 = 0; j0 < nf; j0 += 8) {  // eight of each in flight at once
          float vd[8], vh[8], ve[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const bool ok = j0 + u < nf;
            const int64_t o = base + (int64_t)(ok ? j0 + u : 0) * n_tok;
            vd[u] = ok ? ld_coherent(a.part_dot + o) : 0.f;
            vh[u] = ok ? ld_coherent(a.part_hh + o) : 0.f;
            ve[u] = ok && (KEYP || !F8) ? ld_coherent(a.ee + o) : 0.f;
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            dot += vd[u];
            hh += vh[u];
            ee += ve[u];
          }
        }
        if constexpr (F8) {
          // the token scale of e: k = s_e * (the partials' k / s_e); the memory-side
          // norm takes the quantized row's own sum of squares
          const float se = a.se[t];
          dot *= se;
          ee = KEYP ? ee * se * se : a.e_ssq[t];
        }
        // TK: the epilogues summed e^2 (hh) and the main loops h^2 (ee)
        const float ssq_h = TK ? ee : hh, ssq_k = TK ? hh : ee;
        const float rms_h = sqrtf(ssq_h / (float)d_model + a.eps);
        // the key's norm: of the memory vector (d_mem wide), or KEYP of W_K e (d_model)
        const float rms_e = sqrtf(ssq_k / (float)(KEYP ? d_model : d_mem) + a.eps);
        const float logit = dot / (rms_h * rms_e) * a.inv_sqrt_d;
        const float g = 1.f / (1.f + expf(-logit));
        st_coherent(a.alpha + (int64_t)m * n_tok + t, g);
        if (a.gate_out != nullptr) a.gate_out[(int64_t)m * n_tok + t] = g;
      }
      wait_vm_lgkm0<0>();  // this wave's gate stores have completed
      __syncthreads();     // ... and every other wave's
      if (etid == 0) __hip_atomic_fetch_add(done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    // Stream the tile out: 16-B chunk p = 256 i + tid is token tl = p / 32, physical
    // chunk p % 32; eight LDS reads are issued ahead of their eight stores.
    const bool full = t0 + BT <= n_tok && f0 + BF <= d_model;
    auto stream_out = [&](uint16_t* dst) {
      uint16_t* Ot0 = dst + t0 * d_model;
#pragma unroll
      for (int i0 = 0; i0 < H_LOADS; i0 += 8) {
        u32x4 ov[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int p = (i0 + u) * NTHR + etid;
          const int tl = p / H_CH;
          ov[u] = *reinterpret_cast<const u32x4*>(smem + ENGRAM_QSLOT(tl >> 6) + (tl & 63) * (BF * 2) +
                                                  (p % H_CH) * 16);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int p = (i0 + u) * NTHR + etid;
          const int tl = p / H_CH;
          const int f = f0 + ((p % H_CH) ^ (tl & 31)) * 8;
          if (full || (t0 + tl < n_tok && f < d_model))
            *reinterpret_cast<u32x4*>(Ot0 + (uint32_t)tl * (uint32_t)d_model + f) = ov[u];
        }
      }
    };
    // The epilogue of branch mb: its h tile is in the ring's quarter slots, its gates in
    // s_alpha.
    auto v_epilogue = [&](int mb) {
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const int tl = ewt * WT + j * 32 + (elane & 31);
        const float alpha = s_alpha[tl];
        // all eight cells of this token column are read before any is written, so the
        // reads are issued back to back (a write could alias a later read otherwise)
        u32x4 hv[MF][2];
#pragma unroll
        for (int i = 0; i < MF; ++i)
#pragma unroll
          for (int gp = 0; gp < 2; ++gp)
            hv[i][gp] = *reinterpret_cast<const u32x4*>(
                smem + ENGRAM_HOFF(tl, (ewf * WF + i * 32 + gp * 16 + hsel) >> 3));
        if constexpr (FOLD) {
#pragma unroll
          for (int i = 0; i < MF; ++i) {
#pragma unroll
            for (int gp = 0; gp < 2; ++gp) {
              ENGRAM_WS(ewf * WF + i * 32 + gp * 16 + hsel, ws);
              u32x4 ov;
#pragma unroll
              for (int q = 0; q < 4; ++q)
                ov[q] = pack_bf16(bf16_lo(hv[i][gp][q]) + alpha * (acc[i][j][gp * 8 + 2 * q] * ws[2 * q]),
                                  bf16_hi(hv[i][gp][q]) + alpha * (acc[i][j][gp * 8 + 2 * q + 1] * ws[2 * q + 1]));
              *reinterpret_cast<u32x4*>(smem + ENGRAM_HOFF(tl, (ewf * WF + i * 32 + gp * 16 + hsel) >> 3)) = ov;
            }
          }
        } else {
#pragma unroll
        for (int i = 0; i < MF; ++i) {
#pragma unroll
          for (int gp = 0; gp < 2; ++gp) {
            u32x4 ov;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              ov[q] = pack_bf16(bf16_lo(hv[i][gp][q]) + alpha * acc[i][j][gp * 8 + 2 * q],
                                bf16_hi(hv[i][gp][q]) + alpha * acc[i][j][gp * 8 + 2 * q + 1]);
            *reinterpret_cast<u32x4*>(smem + ENGRAM_HOFF(tl, (ewf * WF + i * 32 + gp * 16 + hsel) >> 3)) = ov;
          }
        }
        }
      }
      lds_barrier();
      ENGRAM_STAMP(12);
      stream_out((uint16_t*)a.out[mb]);
      ENGRAM_STAMP(13);
      if (VALUES && a.vout[mb] != nullptr) {
        // the gated values alpha * v, staged through the same LDS tile
        lds_barrier();
#pragma unroll
        for (int j = 0; j < MT; ++j) {
          const int tl = ewt * WT + j * 32 + (elane & 31);
          const float alpha = s_alpha[tl];
#pragma unroll
          for (int i = 0; i < MF; ++i) {
#pragma unroll
            for (int gp = 0; gp < 2; ++gp) {
              u32x4 ov;
              if constexpr (FOLD) {
                ENGRAM_WS(ewf * WF + i * 32 + gp * 16 + hsel, ws);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                  ov[q] = pack_bf16(alpha * (acc[i][j][gp * 8 + 2 * q] * ws[2 * q]),
                                    alpha * (acc[i][j][gp * 8 + 2 * q + 1] * ws[2 * q + 1]));
              } else {
#pragma unroll
              for (int q = 0; q < 4; ++q)
                ov[q] = pack_bf16(alpha * acc[i][j][gp * 8 + 2 * q], alpha * acc[i][j][gp * 8 + 2 * q + 1]);
              }
              *reinterpret_cast<u32x4*>(smem + ENGRAM_HOFF(tl, (ewf * WF + i * 32 + gp * 16 + hsel) >> 3)) = ov;
            }
          }
        }
        lds_barrier();
        stream_out((uint16_t*)a.vout[mb]);
      }
    };
    if constexpr (!SHAREDV) {
      v_epilogue(m);
    } else {
      for (int mb = 0; mb < a.n_branch; ++mb) {
        if (mb > 0) {
          // branch mb's h tile and gates replace branch mb - 1's, once every read of the
          // tile is done
          lds_barrier();
          // the h-tile loads of the main loop, with every address re-derived here from
          // the opaque thread id (reusing the main loop's would keep them live through it)
          const uint16_t* hb = (const uint16_t*)a.h[mb] + t0 * d_model;
          const int ew = __builtin_amdgcn_readfirstlane(etid >> 6);
          const int blim = (int)(n_tok - 1 - t0);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t dst = (uint32_t)(uintptr_t)(lds_ptr)smem + (uint32_t)(((q0slot + q) % NSLOT) * SLOT_BYTES);
#pragma unroll
            for (int i = 0; i < G_INSTR; ++i) {
              const int blk = ew * G_INSTR + i;
              const int tl = q * 64 + blk * 2 + (elane >> 5);
              const int c = (elane & 31) ^ (tl & 31);
              const int tr = tl < blim ? tl : blim;
              int f = f0 + c * 8;
              f = f < d_model ? f : 0;
              dma16(hb + (uint32_t)tr * (uint32_t)d_model + f, dst + (uint32_t)(blk * 1024));
            }
          }
          float al = gave_up ? __builtin_nanf("")
                             : t0 + etid < n_tok ? ld_coherent(a.alpha + (int64_t)mb * n_tok + t0 + etid) : 0.f;
          if constexpr (F8) al = t0 + etid < n_tok ? al * a.se[t0 + etid] : 0.f;
          wait_vm_lgkm0<0>();
          s_alpha[etid] = al;
          lds_barrier();
        }
        v_epilogue(mb);
      }
    }
  }
  ENGRAM_STAMP(6);
#undef ENGRAM_WS
#undef ENGRAM_HOFF
#undef ENGRAM_QSLOT
}

// The persistent workgroup: claims tiles from its queue until the queue is exhausted.
// smem: the operand ring, then the h tile and the epilogue scratch; between tiles its
// first word broadcasts the claimed tile number.
template <bool VALUES, bool KEYP, bool SHAREDV, bool F8, bool GATHER, bool TK, class GS>
__device__ __forceinline__ void persistent_loop(const GateArgs& a, const GS& gs, char* smem) {
  int* s_tile = reinterpret_cast<int*>(smem);
  const int x = blockIdx.x % NQ;
  int claim = 0;  // thread 0: the tile claimed for after the current one
  if (threadIdx.x == 0) claim = atomicAdd(a.counters + x, 1);
  for (int tl_n = 0;; ++tl_n) {
    ENGRAM_STAMP(0);
    if (threadIdx.x == 0) *s_tile = claim;
    lds_barrier();
    Tile t;
    const bool have = decode_tile<SHAREDV, GATHER, TK>(a, x, *s_tile, t);
    lds_barrier();  // every thread has read the tile number before the ring is refilled
    if (!have) break;
    gate_tile<VALUES, KEYP, SHAREDV, F8, GATHER, TK>(a, gs, t, smem, x, claim, tl_n);
    // LDS free for the next tile.  A full barrier: letting a V tile's 128 KB of output
    // stores drain behind the next tile's operand loads measured 8 % slower than
    // finishing them first.
    __syncthreads();
    ENGRAM_STAMP(7);
  }
}

template <bool VALUES, bool KEYP, bool SHAREDV, bool F8, bool TK>
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gate_persistent_kernel(const GateArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[SMEM_BYTES];
  persistent_loop<VALUES, KEYP, SHAREDV, F8, false, TK>(a, NoGather{}, smem);
}

// engram_lookup_gate: the same kernel reading its memory rows from the tables.
template <bool VALUES, bool KEYP, bool SHAREDV>
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gate_gather_kernel(const GateArgs a, const GatherSrc gs) {
  __shared__ __attribute__((aligned(16))) char smem[SMEM_BYTES];
  persistent_loop<VALUES, KEYP, SHAREDV, false, true, false>(a, gs, smem);
}

// KEYP: the per-feature key gain gq[m][f] * gk[m][f] in fp32 (exact: a product of two
// bf16 values), and the tile queues / done counters cleared; the K tiles read W_K itself.
// Without gains (the FP8 gate with the memory-side key norm, whose gk spans d_mem) only
// the counters are cleared.
__global__ __launch_bounds__(256) void gate_prep_projected_kernel(const GateArgs a, int n_counters, bool gains) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_counters) a.counters[i] = 0;
  if (!gains || i >= (int64_t)a.n_branch * a.d_model) return;
  const int m = (int)(i / a.d_model);
  const int f = (int)(i - (int64_t)m * a.d_model);
  const float gq = __uint_as_float((uint32_t)((const uint16_t*)a.gq[m])[f] << 16);
  const float gk = __uint_as_float((uint32_t)((const uint16_t*)a.gk[m])[f] << 16);
  a.kgain[i] = gq * gk;
}

// One launch before the gate: W'[m][f][c] = bf16(gq[m][f] * W_K[m][f][c] * gk[m][c])
// for every branch (both RMSNorm gains folded into the key weights, one rounding),
// and the tile queues / done counters cleared.
__global__ __launch_bounds__(256) void gate_prep_kernel(const GateArgs a, uint16_t* wk_scaled,
                                                        int64_t n8_per_branch, int n_counters) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_counters) a.counters[i] = 0;
  if (i >= n8_per_branch * a.n_branch) return;
  const int m = (int)(i / n8_per_branch);
  const int64_t k = i - m * n8_per_branch;
  const int f = (int)((k * 8) / a.d_mem);
  const int j = (int)((k * 8) - (int64_t)f * a.d_mem);
  const u32x4 wv = reinterpret_cast<const u32x4*>(a.wk[m])[k];
  const u32x4 gv = *reinterpret_cast<const u32x4*>((const uint16_t*)a.gk[m] + j);
  const float gq = __uint_as_float((uint32_t)((const uint16_t*)a.gq[m])[f] << 16);
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = pack_bf16(gq * bf16_lo(wv[q]) * bf16_lo(gv[q]), gq * bf16_hi(wv[q]) * bf16_hi(gv[q]));
  reinterpret_cast<u32x4*>(wk_scaled)[i] = o;
}

// The same fold for memory-major K tiles, written transposed:
// W'T[m][c][f] = bf16(gq[m][f] * W_K[m][f][c] * gk[m][c]), the same products rounded the same
// way.  One workgroup per 64 x 64 block (d_model and d_mem multiples of 64): each thread
// reads 16 consecutive c of one row f, the block turns in LDS, and each thread writes 16
// consecutive f of one row c.  The counters are cleared grid-stride.
__global__ __launch_bounds__(256) void gate_prep_t_kernel(const GateArgs a, uint16_t* wkt, int n_counters) {
  __shared__ uint16_t blk[64][64 + 2];
  const int tid = threadIdx.x;
  const int64_t gid = ((int64_t)blockIdx.z * gridDim.y * gridDim.x + (int64_t)blockIdx.y * gridDim.x + blockIdx.x) * 256 + tid;
  const int64_t nthreads = (int64_t)gridDim.x * gridDim.y * gridDim.z * 256;
  for (int64_t i = gid; i < n_counters; i += nthreads) a.counters[i] = 0;
  const int m = blockIdx.z;
  const int f0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int d_mem = a.d_mem, d_model = a.d_model;
  {
    const int r = tid >> 2, cs = (tid & 3) * 16;
    const uint16_t* src = (const uint16_t*)a.wk[m] + (int64_t)(f0 + r) * d_mem + c0 + cs;
    const uint16_t* gks = (const uint16_t*)a.gk[m] + c0 + cs;
    const float gq = __uint_as_float((uint32_t)((const uint16_t*)a.gq[m])[f0 + r] << 16);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 wv = reinterpret_cast<const u32x4*>(src)[h];
      const u32x4 gv = reinterpret_cast<const u32x4*>(gks)[h];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t o = pack_bf16(gq * bf16_lo(wv[q]) * bf16_lo(gv[q]), gq * bf16_hi(wv[q]) * bf16_hi(gv[q]));
        blk[r][cs + h * 8 + 2 * q] = (uint16_t)(o & 0xffffu);
        blk[r][cs + h * 8 + 2 * q + 1] = (uint16_t)(o >> 16);
      }
    }
  }
  __syncthreads();
  {
    const int c = tid >> 2, fs = (tid & 3) * 16;
    uint16_t* dst = wkt + (int64_t)m * d_mem * d_model + (int64_t)(c0 + c) * d_model + f0 + fs;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = (uint32_t)blk[fs + h * 8 + 2 * q][c] | ((uint32_t)blk[fs + h * 8 + 2 * q + 1][c] << 16);
      reinterpret_cast<u32x4*>(dst)[h] = o;
    }
  }
}

// One W_V for every branch (the same pointer): W_V e is computed once per tile.
bool shared_wv(const GateArgs& a) {
  bool shared = a.n_branch > 1;
  for (int m = 0; m < a.n_branch; ++m) shared = shared && a.wv[m] == a.wv[0];
  return shared;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// wk_bytes: the gain-folded key weights (the memory-side key norm), or KEYP and fp8 the
// fp32 per-feature key gains.  fp8 adds the codes and scales of both weights (W_V once
// when shared) and of the memory vectors.
struct ScratchLayout {
  size_t wk_bytes, part_bytes, alpha_bytes, counter_bytes, total;
  size_t k8_bytes, v8_bytes, sk_bytes, sv_bytes, e8_bytes, tok_bytes;
  int n_counters;
};

ScratchLayout layout_for(const GateArgs& a, bool fp8, bool prequant) {
  ScratchLayout L;
  L.wk_bytes = (a.key_norm == ENGRAM_KEY_NORM_PROJECTED || fp8 || prequant) ? round256((size_t)a.n_branch * a.d_model * 4)
                                                                 : round256((size_t)a.n_branch * a.d_model * a.d_mem * 2);
  const size_t part_elems = (size_t)a.n_branch * a.n_ftiles * (size_t)a.n_tok;
  L.part_bytes = round256(part_elems * 4);
  L.alpha_bytes = round256((size_t)a.n_branch * (size_t)a.n_tok * 4);
  L.n_counters = NQ + a.n_branch * a.n_ttiles;
  L.counter_bytes = round256((size_t)L.n_counters * 4);
  L.total = L.wk_bytes + 3 * L.part_bytes + L.alpha_bytes + L.counter_bytes;
  L.k8_bytes = L.v8_bytes = L.sk_bytes = L.sv_bytes = L.e8_bytes = L.tok_bytes = 0;
  if (fp8 && !prequant) {
    const size_t n_wv = shared_wv(a) ? 1 : (size_t)a.n_branch;
    L.k8_bytes = round256((size_t)a.n_branch * a.d_model * a.d_mem);
    L.v8_bytes = round256(n_wv * a.d_model * a.d_mem);
    L.sk_bytes = round256((size_t)a.n_branch * a.d_model * 4);
    L.sv_bytes = round256(n_wv * a.d_model * 4);
    L.e8_bytes = round256((size_t)a.n_tok * a.d_mem);
    L.tok_bytes = round256((size_t)a.n_tok * 4);
    L.total += L.k8_bytes + L.v8_bytes + L.sk_bytes + L.sv_bytes + L.e8_bytes + 2 * L.tok_bytes;
  }
  return L;
}

// Test hook: every later gate launch waits for a done count its K tiles never reach,
// bounded by FORCED_SPIN_LIMIT polls, so the give-up path runs (and the kernel ends).
std::atomic<bool> g_force_wait_timeout{false};
// Test hook: the K tiles' form (0 by shape, 1 feature-major, 2 memory-major where it applies).
std::atomic<int> g_key_form{0};

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

size_t gate_bf16_scratch_bytes(GateArgs& a, bool fp8, bool prequant) {
  a.n_ftiles = (a.d_model + BF - 1) / BF;
  a.n_ttiles = (int32_t)((a.n_tok + BT - 1) / BT);
  return layout_for(a, fp8, prequant).total;
}

// `a.part_dot` must point at the scratch block of gate_bf16_scratch_bytes(a) bytes;
// the other scratch pointers are carved from it here.
// prequant, fp8: a.mem, a.se, a.e_ssq, a.wk, a.wv, a.sk and a.sv already hold the codes
// and scales; only the counters and the key gains are prepared here.  prequant, bf16
// with the memory-side key norm: a.wk already holds the gain-folded key weights
// (launch_gate_fold); only the counters are cleared.
void launch_gate_bf16(const GateArgs& a_in, bool fp8, hipStream_t s, bool prequant, const GatherSrc* gs) {
  GateArgs a = a_in;
  const ScratchLayout L = layout_for(a, fp8, prequant);
  const bool shared_v = shared_wv(a);
  char* base = (char*)a_in.part_dot;
  uint16_t* wk_scaled = (uint16_t*)base;
  a.part_dot = (float*)(base + L.wk_bytes);
  a.part_hh = (float*)(base + L.wk_bytes + L.part_bytes);
  a.ee = (float*)(base + L.wk_bytes + 2 * L.part_bytes);
  a.alpha = (float*)(base + L.wk_bytes + 3 * L.part_bytes);
  a.counters = (int32_t*)(base + L.wk_bytes + 3 * L.part_bytes + L.alpha_bytes);

  const bool keyp = a.key_norm == ENGRAM_KEY_NORM_PROJECTED;
  int grid = cu_count() / NQ * NQ;
  if (grid < NQ) grid = NQ;
  // Memory-major K tiles (TK) where they apply (bf16 with the memory-side key norm and the
  // folded weights made here, d_mem < d_model so their partials fit the feature-major
  // layout, d_model a whole number of k-steps) and where there is at least one K tile per
  // CU (a decode step's one token tile would leave most CUs idle behind the longer tiles).
  const int n_ctiles = (a.d_mem + BF - 1) / BF;
  const int form = g_key_form.load(std::memory_order_relaxed);
  const bool tk_ok = !fp8 && !prequant && gs == nullptr && !keyp && a.d_mem < a.d_model && a.d_model % BK == 0;
  const bool tk = tk_ok && form != 1 &&
                  (form == 2 || (int64_t)a.n_ttiles * a.n_branch * n_ctiles >= (int64_t)grid);
  a.n_ktiles = tk ? n_ctiles : a.n_ftiles;
  if (fp8) {
    // the key gains and the counters, then the E4M3 codes: W_K with both gains folded
    // in (memory-side key norm) or as is, W_V, and the memory vectors with their sums
    // of squares
    a.kgain = (float*)base;
    const int64_t gain_work = keyp ? (int64_t)a.n_branch * a.d_model : 0;
    const int64_t work = gain_work > L.n_counters ? gain_work : L.n_counters;
    hipLaunchKernelGGL(gate_prep_projected_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, a,
                       L.n_counters, keyp);
    if (!prequant) {
      char* p = base + L.total - (L.k8_bytes + L.v8_bytes + L.sk_bytes + L.sv_bytes + L.e8_bytes + 2 * L.tok_bytes);
      uint8_t* k8 = (uint8_t*)p;
      uint8_t* v8 = (uint8_t*)(p += L.k8_bytes);
      float* sk = (float*)(p += L.v8_bytes);
      float* sv = (float*)(p += L.sk_bytes);
      uint8_t* e8 = (uint8_t*)(p += L.sv_bytes);
      float* se = (float*)(p += L.e8_bytes);
      float* essq = (float*)(p += L.tok_bytes);
      const size_t wsz = (size_t)a.d_model * a.d_mem;
      for (int m = 0; m < a.n_branch; ++m) {
        launch_quant_rows(a.wk[m], true, a.d_model, a.d_mem, keyp ? nullptr : a.gq[m], keyp ? nullptr : a.gk[m],
                          k8 + m * wsz, sk + (size_t)m * a.d_model, nullptr, s);
        if (m == 0 || !shared_v)
          launch_quant_rows(a.wv[m], true, a.d_model, a.d_mem, nullptr, nullptr, v8 + m * wsz,
                            sv + (size_t)m * a.d_model, nullptr, s);
      }
      launch_quant_rows(a.mem, true, a.n_tok, a.d_mem, nullptr, nullptr, e8, se, essq, s);
      for (int m = 0; m < a.n_branch; ++m) {
        a.wk[m] = k8 + m * wsz;
        a.wv[m] = v8 + (shared_v ? 0 : m) * wsz;
        a.sk[m] = sk + (size_t)m * a.d_model;
        a.sv[m] = sv + (size_t)(shared_v ? 0 : m) * a.d_model;
      }
      a.mem = e8;
      a.se = se;
      a.e_ssq = essq;
    }
  } else if (keyp) {
    a.kgain = (float*)base;
    const int64_t work = (int64_t)a.n_branch * a.d_model > L.n_counters ? (int64_t)a.n_branch * a.d_model
                                                                         : L.n_counters;
    hipLaunchKernelGGL(gate_prep_projected_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, a,
                       L.n_counters, true);
  } else if (prequant) {
    hipLaunchKernelGGL(gate_prep_projected_kernel, dim3((unsigned)((L.n_counters + 255) / 256)), dim3(256), 0, s,
                       a, L.n_counters, false);
  } else if (tk) {
    hipLaunchKernelGGL(gate_prep_t_kernel, dim3((unsigned)(a.d_mem / 64), (unsigned)(a.d_model / 64),
                                               (unsigned)a.n_branch), dim3(256), 0, s, a, wk_scaled, L.n_counters);
    for (int m = 0; m < a.n_branch; ++m) a.wk[m] = wk_scaled + (size_t)m * a.d_model * a.d_mem;
  } else {
    const int64_t n8 = (int64_t)a.d_model * a.d_mem / 8;
    const int64_t work = n8 * a.n_branch > L.n_counters ? n8 * a.n_branch : L.n_counters;
    hipLaunchKernelGGL(gate_prep_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, a,
                       wk_scaled, n8, L.n_counters);
    for (int m = 0; m < a.n_branch; ++m) a.wk[m] = wk_scaled + (size_t)m * a.d_model * a.d_mem;
  }

  const bool forced = g_force_wait_timeout.load(std::memory_order_relaxed);
  a.wait_extra = forced ? 1 : 0;
  a.spin_limit = forced ? FORCED_SPIN_LIMIT : SPIN_LIMIT;
  bool values = false;
  for (int m = 0; m < a.n_branch; ++m) values = values || a.vout[m] != nullptr;
  const dim3 g((unsigned)grid), b(NTHR);
  if (gs != nullptr) {
#define ENGRAM_GATHER_LAUNCH(V_, K_, S_)                                                   \
  if (values == V_ && keyp == K_ && shared_v == S_)                                        \
    hipLaunchKernelGGL((gate_gather_kernel<V_, K_, S_>), g, b, 0, s, a, *gs);
    ENGRAM_GATHER_LAUNCH(false, false, false)
    ENGRAM_GATHER_LAUNCH(false, false, true)
    ENGRAM_GATHER_LAUNCH(false, true, false)
    ENGRAM_GATHER_LAUNCH(false, true, true)
    ENGRAM_GATHER_LAUNCH(true, false, false)
    ENGRAM_GATHER_LAUNCH(true, false, true)
    ENGRAM_GATHER_LAUNCH(true, true, false)
    ENGRAM_GATHER_LAUNCH(true, true, true)
#undef ENGRAM_GATHER_LAUNCH
    return;
  }
  if (tk) {
#define ENGRAM_TK_LAUNCH(V_, S_)                                                           \
  if (values == V_ && shared_v == S_)                                                      \
    hipLaunchKernelGGL((gate_persistent_kernel<V_, false, S_, false, true>), g, b, 0, s, a);
    ENGRAM_TK_LAUNCH(false, false)
    ENGRAM_TK_LAUNCH(false, true)
    ENGRAM_TK_LAUNCH(true, false)
    ENGRAM_TK_LAUNCH(true, true)
#undef ENGRAM_TK_LAUNCH
    return;
  }
#define ENGRAM_GATE_LAUNCH(V_, K_, S_, F_)                                                 \
  if (values == V_ && keyp == K_ && shared_v == S_ && fp8 == F_)                           \
    hipLaunchKernelGGL((gate_persistent_kernel<V_, K_, S_, F_, false>), g, b, 0, s, a);
  ENGRAM_GATE_LAUNCH(false, false, false, false)
  ENGRAM_GATE_LAUNCH(false, false, true, false)
  ENGRAM_GATE_LAUNCH(false, true, false, false)
  ENGRAM_GATE_LAUNCH(false, true, true, false)
  ENGRAM_GATE_LAUNCH(true, false, false, false)
  ENGRAM_GATE_LAUNCH(true, false, true, false)
  ENGRAM_GATE_LAUNCH(true, true, false, false)
  ENGRAM_GATE_LAUNCH(true, true, true, false)
  ENGRAM_GATE_LAUNCH(false, false, false, true)
  ENGRAM_GATE_LAUNCH(false, false, true, true)
  ENGRAM_GATE_LAUNCH(false, true, false, true)
  ENGRAM_GATE_LAUNCH(false, true, true, true)
  ENGRAM_GATE_LAUNCH(true, false, false, true)
  ENGRAM_GATE_LAUNCH(true, false, true, true)
  ENGRAM_GATE_LAUNCH(true, true, false, true)
  ENGRAM_GATE_LAUNCH(true, true, true, true)
#undef ENGRAM_GATE_LAUNCH
}

hipError_t gate_wait_timeouts(int32_t* count, bool reset) {
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbol(count, HIP_SYMBOL(g_gate_wait_timeouts), sizeof(int32_t), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess || !reset) return e;
  const int32_t zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_gate_wait_timeouts), &zero, sizeof(int32_t), 0, hipMemcpyHostToDevice);
}

void set_gate_forced_wait_timeout(bool on) { g_force_wait_timeout.store(on, std::memory_order_relaxed); }

void set_gate_key_form(int form) { g_key_form.store(form, std::memory_order_relaxed); }

void launch_gate_fold(const GateArgs& a_in, uint16_t* const* wk_folded, hipStream_t s) {
  const int64_t n8 = (int64_t)a_in.d_model * a_in.d_mem / 8;
  for (int m = 0; m < a_in.n_branch; ++m) {
    GateArgs a = a_in;  // branch m alone, written to its own output
    a.n_branch = 1;
    a.wk[0] = a_in.wk[m];
    a.gq[0] = a_in.gq[m];
    a.gk[0] = a_in.gk[m];
    hipLaunchKernelGGL(gate_prep_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, a, wk_folded[m], n8,
                       0);
  }
}

void launch_prepare_fp8(const GateArgs& a, uint8_t* const* wk_codes, float* const* wk_scales,
                        uint8_t* const* wv_codes, float* const* wv_scales, hipStream_t s) {
  const bool keyp = a.key_norm == ENGRAM_KEY_NORM_PROJECTED;
  for (int m = 0; m < a.n_branch; ++m) {
    launch_quant_rows(a.wk[m], true, a.d_model, a.d_mem, keyp ? nullptr : a.gq[m], keyp ? nullptr : a.gk[m],
                      wk_codes[m], wk_scales[m], nullptr, s);
    launch_quant_rows(a.wv[m], true, a.d_model, a.d_mem, nullptr, nullptr, wv_codes[m], wv_scales[m], nullptr, s);
  }
}

}  // namespace engram

#ifdef ENGRAM_GATE_TIMELINE
// The timeline build's two extra exports (not in engram.h): copy g_timeline (uint64
// [256][512][16]) to host memory after synchronising the device, and clear it.  0 or -1.
extern "C" int engram_gate_timeline_read(void* host, int64_t bytes) {
  if (host == nullptr || bytes <= 0 || bytes > (int64_t)sizeof(engram::g_timeline)) return -1;
  if (hipDeviceSynchronize() != hipSuccess) return -1;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(engram::g_timeline), (size_t)bytes, 0, hipMemcpyDeviceToHost) ==
                 hipSuccess ? 0 : -1;
}

extern "C" int engram_gate_timeline_clear() {
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(engram::g_timeline)) != hipSuccess) return -1;
  if (hipMemset(p, 0, sizeof(engram::g_timeline)) != hipSuccess) return -1;
  return hipDeviceSynchronize() == hipSuccess ? 0 : -1;
}
#endif
