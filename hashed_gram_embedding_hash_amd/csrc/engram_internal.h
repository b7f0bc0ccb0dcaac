// engram_internal.h -- shared declarations of the HIP library (kernels + C ABI).
// gfx950 only.  Nothing here is visible through include/engram.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/engram.h"

namespace engram {

// ---------------------------------------------------------------- enum arguments
// The int value of an enum argument, which a C caller may have set to any int: read
// through memcpy, because loading a C++ enum object that holds a value outside its
// enumerators' range is undefined behaviour.  Entry points validate this value before
// they use the enum itself.
template <class E>
inline int enum_arg(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "enum arguments are int-sized");
  int v;
  __builtin_memcpy(&v, &e, sizeof v);
  return v;
}

// ---------------------------------------------------------------- errors
engram_status fail(engram_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
engram_status hip_fail(hipError_t e, const char* what);
// Status of the last launch on this thread (hipGetLastError), mapped to engram_status.
engram_status check_launch(const char* what);

// ---------------------------------------------------------------- compress
void launch_compress(const int32_t* raw, int64_t n, const int32_t* map, int32_t vocab, int32_t* out,
                     int32_t* err_count, hipStream_t s);

// ---------------------------------------------------------------- hash
struct HashArgs {
  uint64_t mult[ENGRAM_MAX_TABLES][ENGRAM_MAX_ORDER];  // per table, per position in the gram
  uint64_t barrett[ENGRAM_MAX_TABLES];                  // floor((2^64 - 1) / rows)
  uint32_t rows[ENGRAM_MAX_TABLES];
  int32_t order[ENGRAM_MAX_TABLES];                     // n of the table's order
  const int32_t* ids;
  int32_t* idx;
  // compress fused in (engram_compress_hash): ids are raw ids mapped through `map` as
  // they are staged; the window's canonical ids go to ids_out when it is set
  const int32_t* map;   // null: ids are canonical already
  int32_t* ids_out;
  int32_t* err_count;
  int64_t ld, t_begin, t_count;
  int32_t n_tables, max_order, pad_id, batch, vocab;
};
void launch_hash(const HashArgs& a, hipStream_t s);

// h mod M for a prime M < 2^31, with the Barrett constant m = floor((2^64 - 1) / M):
// q = mulhi(h, m) is floor(h / M) or one less, so one conditional subtraction remains.
__device__ __forceinline__ uint32_t mod_barrett(uint64_t h, uint32_t M, uint64_t m) {
  const uint64_t q = __umul64hi(h, m);
  const uint64_t r = h - q * (uint64_t)M;
  return (uint32_t)(r >= M ? r - M : r);
}


// ---------------------------------------------------------------- gather / prefetch
struct GatherArgs {
  const char* table[ENGRAM_MAX_TABLES];  // device-accessible base of each table
  int64_t rows[ENGRAM_MAX_TABLES];
  const int32_t* idx;
  char* out;
  int32_t* err_count;
  int64_t n_tok;
  int32_t n_tables;
  int32_t chunks_per_row;  // row bytes / 16
};
// `host_source`: the tables are pinned host memory read over PCIe (launch tuned for that).
void launch_gather(const GatherArgs& a, bool host_source, hipStream_t s);
// engram_lookup: the hash kernel's staging and index computation for a block of
// positions, then the gather of their rows, in one kernel (h.idx may be null: the
// indices then stay in LDS; g.idx is unused).  With q8 (bf16 rows only), each
// position's memory vector is quantized to E4M3 instead of stored (g.out unused).
struct Q8Out {
  uint8_t* codes;  // [positions][d_mem]
  float* scales;   // [positions]
  float* sumsq;    // [positions] or null
};
void launch_lookup(const HashArgs& h, const GatherArgs& g, const Q8Out* q8, hipStream_t s);
// prefetch from host tables through the HBM row cache (table: [n_tables][2^log2_slots])
void launch_prefetch_cached(const GatherArgs& a, const int2* table, int log2_slots, const char* cache_rows,
                            int32_t* hits, hipStream_t s);

// ---------------------------------------------------------------- FP8 quantization
// per-row E4M3 codes and fp32 scales of src [rows][cols] (cols % 16 == 0); grow [rows] /
// gcol [cols] optional gains folded in first; sumsq [rows] optional
void launch_quant_rows(const void* src, bool bf16, int64_t rows, int32_t cols, const void* grow, const void* gcol,
                       uint8_t* codes, float* scales, float* sumsq, hipStream_t s);

// ---------------------------------------------------------------- gate
struct GateArgs {
  const void* mem;
  const void* h[ENGRAM_MAX_BRANCHES];
  const void* wk[ENGRAM_MAX_BRANCHES];
  const void* wv[ENGRAM_MAX_BRANCHES];
  const void* gq[ENGRAM_MAX_BRANCHES];
  const void* gk[ENGRAM_MAX_BRANCHES];
  void* out[ENGRAM_MAX_BRANCHES];
  void* vout[ENGRAM_MAX_BRANCHES];  // gated values alpha * v, or null per branch
  float* gate_out;   // [n_branch][n_tok] or null
  float* part_dot;   // scratch: [n_branch][n_ftiles][n_tok] (the first n_ktiles of each branch used)
  float* part_hh;    // scratch: [n_branch][n_ftiles][n_tok] partial sums of h^2 (memory-major: e^2)
  float* ee;         // scratch: [n_branch][n_ftiles][n_tok] partial sums of e^2 (memory-major: h^2)
  float* alpha;      // scratch: [n_branch][n_tok] gates, published by the last K tile of a token tile
  int32_t* counters; // scratch: per-queue tile heads, then per-(branch, token tile) done counts
  float* kgain;      // scratch, projected key norm: [n_branch][d_model] gq * gk
  int64_t n_tok;
  int32_t d_mem, d_model, n_branch, n_ftiles, n_ttiles;
  int32_t key_norm;  // engram_key_norm
  float eps, inv_sqrt_d;
  // FP8 projections: per branch the per-feature scales of the key and value weight codes
  // ([d_model] each; with one shared W_V, branch 0's), and per token the scale and the
  // sum of squares of the dequantized memory vector
  const float* se;
  const float* e_ssq;
  const float* sk[ENGRAM_MAX_BRANCHES];
  const float* sv[ENGRAM_MAX_BRANCHES];
  // the V tiles' bounded wait: the done count it needs is n_ktiles + 1 + wait_extra
  // (wait_extra is 0 except under the forced-timeout test hook), polled at most
  // spin_limit times (set by launch_gate_bf16)
  int32_t wait_extra, spin_limit;
  // K tiles per (branch, token tile), set by launch_gate_bf16: n_ftiles, or with the key
  // phase contracted over d_model (memory-major K tiles) ceil(d_mem / 256) <= n_ftiles
  int32_t n_ktiles;
};
// engram_lookup_gate: the bf16 gate reads its memory rows straight from the tables.
// Position p's row in table b starts at tab[b] + z * cpr * 16 bytes, with
// z = (XOR_{j < order[b]} x'_{t-j} * mult[b][j] mod 2^64) mod rows[b] and the canonical
// ids x'_{t-j} of the position in ids[p] (j = 0..3, the pad id before a sequence's
// start).  The memory vector is the concatenation of the rows (cpr 16-byte chunks each,
// cpr >= 8, n_tables * cpr * 8 == d_mem).
struct GatherSrc {
  const int4* ids;  // [n_tok]
  const char* tab[ENGRAM_MAX_TABLES];
  uint64_t mult[ENGRAM_MAX_TABLES][ENGRAM_MAX_ORDER];
  uint64_t barrett[ENGRAM_MAX_TABLES];  // floor((2^64 - 1) / rows)
  uint32_t rows[ENGRAM_MAX_TABLES];
  int32_t order[ENGRAM_MAX_TABLES];
  int32_t n_tables, cpr;
};
// The ids GatherSrc::ids holds, for positions [batch][t_count] of the hashing window of h
// (compression through h.map as in engram_compress_hash, counted in h.err_count and
// written to h.ids_out when set).
void launch_gate_ids(const HashArgs& h, int4* ids, hipStream_t s);

// bf16 path: returns the scratch bytes it needs for these shapes (and sets a.n_ftiles).
// launch_gate_bf16 expects a.part_dot to point at a scratch block of that size.  With
// fp8, the projections run on E4M3 codes that it quantizes first (d_mem % 128 == 0).
// With gs (bf16 only), the memory rows come from the tables gs describes (a.mem unused).
size_t gate_bf16_scratch_bytes(GateArgs& a, bool fp8, bool prequant = false);
void launch_gate_bf16(const GateArgs& a, bool fp8, hipStream_t s, bool prequant = false,
                      const GatherSrc* gs = nullptr);
// The FP8 weights as the gate uses them: E4M3 codes of W_K (with the memory-side key
// norm, of gq[f] * W_K[f][c] * gk[c] formed in fp32) and of W_V, per branch, with their
// per-feature scales (one launch of the quantizer per matrix).
void launch_prepare_fp8(const GateArgs& a, uint8_t* const* wk_codes, float* const* wk_scales,
                        uint8_t* const* wv_codes, float* const* wv_scales, hipStream_t s);
// The gain-folded key weights of the bf16 gate (memory-side key norm), per branch:
// wk_folded[m][f][c] = bf16(gq[m][f] * wk[m][f][c] * gk[m][c]), as every bf16 call
// without prepared weights computes them (uses a.wk, a.gq, a.gk, d_mem, d_model, n_branch).
void launch_gate_fold(const GateArgs& a, uint16_t* const* wk_folded, hipStream_t s);
void launch_gate_f32(const GateArgs& a, hipStream_t s);
// Reads (and with reset zeroes) the current device's count of V-tile wavefronts whose
// wait for the gates ran out; synchronizes the device first.
hipError_t gate_wait_timeouts(int32_t* count, bool reset);
// Test hook behind engram_debug_force_gate_timeout.
void set_gate_forced_wait_timeout(bool on);
// Test hook behind engram_debug_gate_key_form: 0 chooses the K tiles' form by shape,
// 1 always feature-major, 2 memory-major wherever that form applies.
void set_gate_key_form(int form);
// engram_gate_forward_noalloc's bf16 launch on the library's fixed device array (a is
// checked and filled by the caller; the scratch pointer is set here).
engram_status gate_forward_noalloc(const char* fn, GateArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- FP8 (E4M3) encoding
// Shared by the quantization kernels and the quantizing lookup (their codes must agree).
// The codes of four quotients x / s, packed little-endian.  The library's code of a
// value is the nearest E4M3 value, ties to the even code, magnitudes at or above 448
// saturated to 448 (see engram_quantize_fp8 in engram.h).  gfx950's conversion
// instruction rounds exactly so for every finite fp32 input below 464 in magnitude
// (checked exhaustively); the clamp makes it saturate where a quotient could exceed
// that (an fp32 row whose maximum underflows the scale to zero).  Inputs are finite.
__device__ __forceinline__ uint32_t e4m3_pack4(float q0, float q1, float q2, float q3) {
  auto sat = [](float q) { return fminf(fmaxf(q, -448.0f), 448.0f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(q0), sat(q1), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(q2), sat(q3), w, true);
  return (uint32_t)w;
}

// The value of byte B of a packed word of codes (exact).
template <int B>
__device__ __forceinline__ float e4m3_byte(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, B);
}

// The sum of squares of the four dequantized values d = value(code) * s of a word.
__device__ __forceinline__ float sumsq4(uint32_t w, float s) {
  const float d0 = e4m3_byte<0>(w) * s, d1 = e4m3_byte<1>(w) * s;
  const float d2 = e4m3_byte<2>(w) * s, d3 = e4m3_byte<3>(w) * s;
  return ((d0 * d0 + d1 * d1) + d2 * d2) + d3 * d3;
}

// ---------------------------------------------------------------- short convolution
struct ConvArgs {
  const void* value;  // [batch * seq][d_model] gated values
  void* out;          // same shape, updated in place
  const void* w;      // [d_model][taps]
  const void* gamma;  // [d_model]
  void* inv;          // scratch [batch * seq]: 1 / rms of each value row (fp32 for bf16 values, fp64 for fp32)
  int64_t seq;
  int32_t batch, d_model, taps, dil;
  float eps;
};
// scratch bytes the convolution needs (its inv array); a.inv must point at that many
size_t conv_scratch_bytes(const ConvArgs& a, bool bf16);
void launch_conv(const ConvArgs& a, bool bf16, hipStream_t s);

}  // namespace engram
