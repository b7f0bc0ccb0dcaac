/*
 * engram.h -- C ABI of the Engram forward pass on AMD Instinct MI355X (gfx950).
 *
 * The module computed here is defined in "Conditional Memory via Scalable
 * Lookup: A New Axis of Sparsity for Large Language Models" (DeepSeek-AI and
 * Peking University):
 *   section 2.2  tokenizer compression, suffix n-grams, multi-head hashing into
 *                prime-sized tables (Eq. 1), concatenated memory vector (Eq. 2);
 *   section 2.3  context-aware gating (Eq. 3-4), gated value and residual add;
 *                the short depthwise causal convolution over the gated values
 *                (Eq. 5);
 *   section 2.4  several branches sharing one lookup (Eq. 6);
 *   section 2.5 / Figure 2(b) and section 6.4  host-memory offload with
 *                prefetch of the rows whose addresses are known in advance.
 * The order of operations in the gate (key = W_K * RMSNorm(memory)) follows the
 * context_aware_gating pseudocode of the review page "Engram: LLM에 '기억의
 * 서랍'을 달아주다" (koala.ai.kr).
 *
 * Conventions for every entry point
 *   - Pointers named "device" must be device memory (hipMalloc or any
 *     allocator over it, e.g. torch CUDA tensors); "host" pointers are ordinary
 *     host memory read during the call.  Arrays of pointers (tables, branch
 *     buffers) are host arrays of device pointers.
 *   - All work is enqueued asynchronously on `stream` (0 = the null stream);
 *     the call returns after enqueueing.  Outputs are valid once the stream
 *     reaches that point.
 *   - Ownership: the library never frees or keeps caller buffers.  The gate
 *     and the convolution share one grow-only scratch buffer per device (a few
 *     MB to a few hundred MB, by shape), allocated stream-ordered on first use
 *     and held until the process ends; a call on a different stream than the
 *     previous user of the scratch first waits for that call's work on it.  A
 *     call that needs more scratch than any call before it replaces the buffer
 *     (the old one is freed in stream order), so a HIP graph captured earlier
 *     must not be replayed after such a call: capture after a call of the
 *     largest shape the graph will be used with.
 *   - Errors: arguments are validated on the host before anything is enqueued;
 *     a non-OK status means nothing was enqueued (ENGRAM_ERR_INVALID_ARG,
 *     ENGRAM_ERR_UNSUPPORTED) or a HIP call failed (ENGRAM_ERR_HIP).
 *     engram_last_error() returns a message for the calling thread's last
 *     non-OK status.  Data errors found on the device (an out-of-range id or
 *     row index) never abort: the element is written as documented and an
 *     optional device counter is incremented.
 *   - Calls are thread-safe; calls on different streams may run concurrently.
 */
#ifndef ENGRAM_H
#define ENGRAM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum engram_status {
  ENGRAM_OK = 0,
  ENGRAM_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size or range     */
  ENGRAM_ERR_UNSUPPORTED = 2, /* valid request outside the implemented shapes    */
  ENGRAM_ERR_HIP = 3          /* a HIP runtime call or a kernel launch failed    */
} engram_status;

typedef enum engram_dtype {
  ENGRAM_F32 = 0, /* IEEE binary32 */
  ENGRAM_BF16 = 1 /* bfloat16 (top 16 bits of binary32), round-to-nearest-even on output */
} engram_dtype;

/* Where the key's RMSNorm sits in the context-aware gate. */
typedef enum engram_key_norm {
  /* k = W_K * RMSNorm_gk(e), gk over d_mem: the context_aware_gating pseudocode of the
   * review page (koala.ai.kr) */
  ENGRAM_KEY_NORM_MEMORY = 0,
  /* k = RMSNorm_gk(W_K * e), gk over d_model: the paper's Eq. (4) and Eq. (6) */
  ENGRAM_KEY_NORM_PROJECTED = 1
} engram_key_norm;

/* Size of the fixed device array behind engram_gate_forward_noalloc (128 MiB). */
#define ENGRAM_NOALLOC_SCRATCH_BYTES (128u << 20)

/* Limits of this implementation. */
#define ENGRAM_MAX_TABLES 32   /* n_orders * heads                       */
#define ENGRAM_MAX_ORDER 4     /* largest n-gram order                   */
#define ENGRAM_MAX_BRANCHES 8  /* gating branches per call               */
#define ENGRAM_CONV_MAX_TAPS 8       /* kernel size of the short convolution  */
#define ENGRAM_CONV_MAX_DILATION 16  /* its dilation                          */

/* Message for the calling thread's last non-OK status ("" if none). */
const char* engram_last_error(void);

/* Library version string. */
const char* engram_version(void);

/*
 * Tokenizer compression -- section 2.2 ("tokenizer compression"): each raw id
 * is mapped through the precomputed surjection P to its canonical id.
 *   out[i] = map[raw[i]]  if 0 <= raw[i] < vocab,  else -1 (and *err_count += 1).
 * raw, out: device int32[n] (may alias).  map: device int32[vocab].
 * err_count: device int32 counter or NULL; it is incremented, never cleared.
 * n == 0 is a no-op.  Errors: INVALID_ARG for n < 0, vocab <= 0 or null pointers.
 */
engram_status engram_compress(const int32_t* raw, int64_t n, const int32_t* map, int32_t vocab,
                              int32_t* out, int32_t* err_count, hipStream_t stream);

/*
 * Multi-head hashing of suffix n-grams -- section 2.2, Eq. (1).
 * ids: device int32 [batch][ld] canonical ids, row-major.  For every row b,
 * position t in [t_begin, t_begin + t_count), order index o (n = orders[o]) and
 * head k < heads:
 *   h = XOR_{j=0}^{n-1} ( (uint64) x'_{t-j} * mult[o][k][j]  mod 2^64 )
 *   idx[b*t_count + (t - t_begin)][o*heads + k] = h mod rows[o*heads + k]
 * where x'_{t-j} is pad_id when t-j < 0 (n-grams never cross rows).  The id is
 * taken as its 32-bit unsigned pattern.
 * orders: host int32[n_orders], each 1..ENGRAM_MAX_ORDER.
 * mult:   host uint64[n_orders][heads][max(orders)] multipliers (entries j >= n unused).
 * rows:   host uint32[n_orders*heads] table sizes, each in [1, 2^31).
 * idx:    device int32 [batch*t_count][n_orders*heads] (order-major, head-minor
 *         columns: the concatenation order of Eq. (2)).
 * Requires 0 <= t_begin, t_begin + t_count <= ld, n_orders*heads <= ENGRAM_MAX_TABLES.
 * batch == 0 or t_count == 0 is a no-op.
 */
engram_status engram_hash(const int32_t* ids, int32_t batch, int64_t ld, int64_t t_begin,
                          int64_t t_count, const int32_t* orders, int32_t n_orders, int32_t heads,
                          const uint64_t* mult, const uint32_t* rows, int32_t pad_id,
                          int32_t* idx, hipStream_t stream);

/*
 * Tokenizer compression fused into the hashing -- section 2.2: exactly
 * engram_compress of raw into canonical ids followed by engram_hash of those ids,
 * in one kernel that maps each raw id through `map` as it loads it.
 * raw: device int32 [batch][ld] raw ids.  map, vocab: as for engram_compress (an
 * id outside [0, vocab) becomes -1 and counts once in *err_count, for positions
 * in the window).  ids_out: device int32 [batch][ld] receiving the canonical ids
 * of the window's positions, or NULL.  All other arguments and idx as for
 * engram_hash.
 */
engram_status engram_compress_hash(const int32_t* raw, int32_t batch, int64_t ld, int64_t t_begin,
                                   int64_t t_count, const int32_t* map, int32_t vocab, const int32_t* orders,
                                   int32_t n_orders, int32_t heads, const uint64_t* mult, const uint32_t* rows,
                                   int32_t pad_id, int32_t* ids_out, int32_t* idx, int32_t* err_count,
                                   hipStream_t stream);

/*
 * Table lookup and concatenation -- section 2.2, Eq. (1)-(2):
 *   out[t][b*w : (b+1)*w] = tables[b][idx[t][b]][0 : w]     (bitwise copy)
 * idx:    device int32 [n_tok][n_tables].
 * tables: host array of n_tables device pointers; table b is row-major
 *         [rows[b]][w] of `dtype`, 16-byte aligned.
 * rows:   host int64[n_tables] row counts.  An index outside [0, rows[b]) yields
 *         a zero block and increments *err_count (device int32, or NULL).
 * out:    device [n_tok][n_tables*w] of `dtype`, 16-byte aligned.
 * Requires w * sizeof(dtype) to be a multiple of 16 (UNSUPPORTED otherwise).
 */
engram_status engram_gather(const int32_t* idx, int64_t n_tok, int32_t n_tables,
                            const void* const* tables, const int64_t* rows, int32_t w,
                            engram_dtype dtype, void* out, int32_t* err_count, hipStream_t stream);

/*
 * Compression, hashing and lookup in one call -- section 2.2, Eq. (1)-(2): exactly
 * engram_compress_hash of raw into canonical ids and indices, followed by
 * engram_gather of those indices from `tables`, in one kernel that keeps the
 * indices on chip.
 * raw, batch, ld, t_begin, t_count, map, vocab, orders, n_orders, heads, mult,
 *   pad_id, ids_out: as for engram_compress_hash; map may be NULL (raw holds
 *   canonical ids already; vocab is then ignored).
 * rows:   host uint32[n_orders*heads]: the prime row count of each table, the
 *         modulus of its hash.
 * tables, w, dtype: as for engram_gather; table b has rows[b] rows.
 * idx_out: device int32 [batch*t_count][n_orders*heads] receiving the indices (the
 *         engram_hash result), or NULL.
 * out:    device [batch*t_count][n_orders*heads*w] of dtype, 16-byte aligned: row
 *         b*t_count + p is position t_begin + p of sequence b.
 * err_count: device int32, incremented once per window position whose raw id is
 *         outside [0, vocab) (with map), or NULL.
 * Requires what engram_compress_hash and engram_gather require.
 */
engram_status engram_lookup(const int32_t* raw, int32_t batch, int64_t ld, int64_t t_begin, int64_t t_count,
                            const int32_t* map, int32_t vocab, const int32_t* orders, int32_t n_orders,
                            int32_t heads, const uint64_t* mult, const uint32_t* rows, int32_t pad_id,
                            const void* const* tables, int32_t w, engram_dtype dtype, int32_t* ids_out,
                            int32_t* idx_out, void* out, int32_t* err_count, hipStream_t stream);

/*
 * The lookup with its memory vectors quantized -- section 2.2, Eq. (1)-(2), and the
 * FP8 projections of section 2.4: exactly engram_lookup on bf16 tables followed by
 * engram_quantize_fp8 of its output with sums of squares, in one kernel that never
 * stores the bf16 vectors (the input of engram_gate_forward_fp8q).
 * raw .. w, ids_out, idx_out, err_count: as for engram_lookup, tables in bf16.
 * codes:  device uint8 [batch*t_count][n_orders*heads*w], 16-byte aligned.
 * scales: device float [batch*t_count]: each vector's scale.
 * sumsq:  device float [batch*t_count]: each vector's sum of squares of its dequantized
 *         values (summed in a fixed order, but not in engram_quantize_fp8's), or NULL.
 */
engram_status engram_lookup_fp8(const int32_t* raw, int32_t batch, int64_t ld, int64_t t_begin, int64_t t_count,
                                const int32_t* map, int32_t vocab, const int32_t* orders, int32_t n_orders,
                                int32_t heads, const uint64_t* mult, const uint32_t* rows, int32_t pad_id,
                                const void* const* tables, int32_t w, int32_t* ids_out, int32_t* idx_out,
                                uint8_t* codes, float* scales, float* sumsq, int32_t* err_count, hipStream_t stream);

/*
 * Context-aware gating -- section 2.3, Eq. (3)-(4), the gated value and the
 * residual update; section 2.4, Eq. (6) for branches m < n_branch sharing `mem`
 * (every branch has its own W_K, W_V and gains; the paper's shared W_V is the
 * case of equal pointers):
 *   q     = RMSNorm_{gq[m]}(h[m]_t),  RMSNorm_g(x) = x / sqrt(mean(x^2) + eps) * g
 *   k     = Wk[m] * RMSNorm_{gk[m]}(mem_t)      (key_norm ENGRAM_KEY_NORM_MEMORY)
 *         = RMSNorm_{gk[m]}(Wk[m] * mem_t)      (key_norm ENGRAM_KEY_NORM_PROJECTED)
 *   v     = Wv[m] * mem_t
 *   alpha = sigmoid( q . k / sqrt(d_model) )
 *   out[m]_t = h[m]_t + alpha * v
 * mem:   device [n_tok][d_mem].   h[m], out[m]: device [n_tok][d_model]; out[m]
 *        may equal h[m] (in place).  Wk[m], Wv[m]: device [d_model][d_mem]
 *        row-major (output x input).  gq[m]: device [d_model]; gk[m]: [d_mem]
 *        (ENGRAM_KEY_NORM_MEMORY) or [d_model] (ENGRAM_KEY_NORM_PROJECTED).
 *        All of `dtype`, 16-byte aligned.
 * gate_out: device float32 [n_branch][n_tok] receiving alpha, or NULL.
 * value_out: NULL, or a host array of n_branch pointers, each NULL or device
 *        [n_tok][d_model] of `dtype` (16-byte aligned, overlapping neither h[m]
 *        nor out[m]) receiving the gated value alpha * v, rounded to `dtype`:
 *        the input of the short convolution (engram_conv_forward).
 * Arithmetic: bf16 products with fp32 accumulation on the matrix cores, fp32
 * elsewhere; with ENGRAM_KEY_NORM_MEMORY the bf16 path folds both gains into a
 * copy of W_K rounded once to bf16, and sums the logit's dot product in fp32 over
 * feature-major or memory-major key tiles, chosen by shape (engram_debug_gate_key_form):
 * the results are reproducible bit for bit for given shapes.  ENGRAM_F32 (fp32 storage)
 * computes every sum, norm and the sigmoid in fp64 and rounds each output to fp32 once.
 * Shapes: ENGRAM_BF16 needs d_mem % 64 == 0 and d_model % 32 == 0, d_model * d_mem
 * < 2^32 and n_tok < 2^31, and at most 2^29 tiles of 256 tokens x 256 features over
 * all branches; ENGRAM_F32 needs d_mem <= 16384 (d_mem + d_model <= 16384 with
 * ENGRAM_KEY_NORM_PROJECTED) and n_tok < 2^31.  Larger
 * requests return ENGRAM_ERR_UNSUPPORTED.  n_tok == 0 is a no-op.
 * Cross-workgroup wait: in the bf16 and FP8 paths the value tiles of a token tile
 * wait, bounded, for its gates (published by the key tiles of the same launch, which
 * always run first).  A wavefront whose wait runs out writes NaN for its tokens'
 * outputs and is counted; engram_gate_wait_timeouts reads that count.
 */
engram_status engram_gate_forward(const void* mem, int64_t n_tok, int32_t d_mem, int32_t d_model,
                                  int32_t n_branch, const void* const* h, const void* const* wk,
                                  const void* const* wv, const void* const* gq,
                                  const void* const* gk, float eps, engram_dtype dtype,
                                  engram_key_norm key_norm, void* const* out, float* gate_out,
                                  void* const* value_out, hipStream_t stream);

/*
 * engram_gate_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): same
 * arguments, same results bit for bit, but no allocation of any kind.  The bf16 path's
 * scratch (gain-folded key weights, partial sums, gates, work-queue counters) is a
 * fixed device array of ENGRAM_NOALLOC_SCRATCH_BYTES that each device the library runs
 * on holds until the process ends; shapes needing more return ENGRAM_ERR_UNSUPPORTED:
 *   n_branch * d_model * d_mem * 2 + 12 * n_branch * ceil(d_model / 256) * n_tok
 *   + 4 * n_branch * n_tok (+ a few KB of counters) bytes, each term rounded up to 256.
 * (The large workload -- 262,144 tokens, d_model 4096, d_mem 1280, 2 branches -- needs
 * 124 MB.)  All calls on one device share the array and it keeps the last call's
 * contents: calls that overlap on one device race, so order them (one stream, or events).
 * The first call on a device looks the array's address up (hipGetSymbolAddress); a
 * failure there is ENGRAM_ERR_HIP.  ENGRAM_F32 uses no scratch and behaves as
 * engram_gate_forward.
 */
engram_status engram_gate_forward_noalloc(const void* mem, int64_t n_tok, int32_t d_mem, int32_t d_model,
                                          int32_t n_branch, const void* const* h, const void* const* wk,
                                          const void* const* wv, const void* const* gq, const void* const* gk,
                                          float eps, engram_dtype dtype, engram_key_norm key_norm, void* const* out,
                                          float* gate_out, void* const* value_out, hipStream_t stream);

/*
 * Health of the gate's cross-workgroup wait (see engram_gate_forward): *count receives
 * the number of value-tile wavefronts on the current device whose bounded wait for
 * their gates ran out since the library was loaded or the count was last reset; their
 * outputs were written as NaN.  0 in normal operation.  reset != 0 zeroes the count
 * after reading it.  Synchronizes the current device (hipDeviceSynchronize) first.
 * Errors: INVALID_ARG for a null count; HIP if a runtime call fails.
 */
engram_status engram_gate_wait_timeouts(int32_t* count, int32_t reset);

/*
 * Test hook for the path above, for tests that must see it run: with on != 0, every
 * later bf16 or FP8 gate launch (any device, until called again with 0) waits for a
 * done count its key tiles never reach, giving up after 64 polls, so every value-tile
 * wavefront writes NaN and is counted; every kernel still completes.  Never set it
 * outside such a test.  Always returns ENGRAM_OK.
 */
engram_status engram_debug_force_gate_timeout(int32_t on);

/*
 * Test hook: the form of the key tiles of engram_gate_forward and
 * engram_gate_forward_noalloc (bf16, memory-side key norm).  The logit's dot product
 * q . k is the same sum in two tilings -- section 2.3, Eq. (4):
 *   feature-major  sum_f h_f (W_K' e)_f, over d_model/256 tiles of 256 features, each
 *                  contracting over d_mem;
 *   memory-major   sum_c e_c (W_K'^T h)_c, over d_mem/256 tiles of 256 memory
 *                  dimensions, each contracting over d_model (fewer, longer tiles).
 * The two differ only in the fp32 rounding order of that sum.  form 0 (the default)
 * chooses by shape: memory-major when d_mem < d_model, d_model % 64 == 0 and there are at
 * least as many memory-major tiles as compute units; feature-major otherwise.  1 forces feature-major, 2 memory-major wherever it applies.  The setting is process-wide and
 * read at each launch.  INVALID_ARG for another form; never set it outside tests and
 * measurements.
 */
engram_status engram_debug_gate_key_form(int32_t form);

/*
 * The bf16 gate with the memory-side key norm, its weights prepared once -- section
 * 2.3, Eq. (3)-(4), as engram_gate_forward computes them.  With this key placement
 * q . k = sum_f h_f gq_f (W_K diag(gk) e)_f / (rms(h) rms(e)), so both RMSNorm gains fold
 * into the key weights; engram_gate_forward folds them on every call, and these two
 * calls let constant weights be folded once.
 * engram_gate_prepare: wk_folded[m][f][c] = bf16(gq[m][f] * wk[m][f][c] * gk[m][c]),
 *   computed in fp32 and rounded to nearest even.
 *   wk, wk_folded: host arrays of n_branch device pointers to [d_model][d_mem] bf16
 *   (wk_folded caller-allocated, 16-byte aligned).  gq[m]: [d_model]; gk[m]: [d_mem] bf16.
 * engram_gate_forward_prepared: engram_gate_forward(dtype ENGRAM_BF16, key_norm
 *   ENGRAM_KEY_NORM_MEMORY) with W_K replaced by wk_folded and no gains.  Its key tiles are
 *   always feature-major (see engram_debug_gate_key_form): its outputs are bit-identical
 *   to that call's with the weights and gains that were folded and that form (the form
 *   engram_gate_forward chooses by itself for token counts that give each compute unit
 *   fewer than two key tiles, as in decode steps).  The other arguments are as for
 *   engram_gate_forward.
 * Both require d_mem % 64 == 0 and d_model % 32 == 0 (ENGRAM_ERR_UNSUPPORTED otherwise).
 */
engram_status engram_gate_prepare(int32_t d_mem, int32_t d_model, int32_t n_branch, const void* const* wk,
                                  const void* const* gq, const void* const* gk, void* const* wk_folded,
                                  hipStream_t stream);
engram_status engram_gate_forward_prepared(const void* mem, int64_t n_tok, int32_t d_mem, int32_t d_model,
                                           int32_t n_branch, const void* const* h, const void* const* wk_folded,
                                           const void* const* wv, float eps, void* const* out, float* gate_out,
                                           void* const* value_out, hipStream_t stream);

/*
 * Lookup and gate in one pass, the memory vectors never stored -- section 2.2, Eq. (1)-(2)
 * feeding section 2.3, Eq. (3)-(4) (and section 2.4, Eq. (6) for several branches):
 * exactly engram_lookup of raw (bf16 tables) into memory vectors e [batch*t_count][d_mem],
 * d_mem = n_orders*heads*w, followed by engram_gate_forward(e, batch*t_count, d_mem, ...,
 * ENGRAM_BF16, key_norm, ...); the outputs are bit-identical to those two calls' with
 * feature-major key tiles (see engram_debug_gate_key_form: where engram_gate_forward would
 * choose memory-major ones, the two differ in the fp32 rounding order of the logit).  The
 * gate's matrix-core kernel hashes each token's n-grams itself and loads the table rows
 * straight into its operand tiles, so e makes no round trip through device memory.
 * raw .. w, ids_out, err_count: as for engram_lookup (dtype ENGRAM_BF16; no index output).
 * d_model .. value_out: as for engram_gate_forward with dtype ENGRAM_BF16 and
 *         n_tok = batch * t_count; gk[m] is [d_mem] for ENGRAM_KEY_NORM_MEMORY.
 * Requires what engram_lookup and engram_gate_forward require, and w >= 64
 * (UNSUPPORTED otherwise).  Uses the library's per-device scratch as
 * engram_gate_forward does, plus 16 bytes per token.  batch == 0 or t_count == 0 is a
 * no-op.
 */
engram_status engram_lookup_gate(const int32_t* raw, int32_t batch, int64_t ld, int64_t t_begin, int64_t t_count,
                                 const int32_t* map, int32_t vocab, const int32_t* orders, int32_t n_orders,
                                 int32_t heads, const uint64_t* mult, const uint32_t* rows, int32_t pad_id,
                                 const void* const* tables, int32_t w, int32_t d_model, int32_t n_branch,
                                 const void* const* h, const void* const* wk, const void* const* wv,
                                 const void* const* gq, const void* const* gk, float eps, engram_key_norm key_norm,
                                 void* const* out, float* gate_out, void* const* value_out, int32_t* ids_out,
                                 int32_t* err_count, hipStream_t stream);

/*
 * Short depthwise causal convolution -- section 2.3, Eq. (5): with V~ the
 * gated values of one sequence (value_out of engram_gate_forward), the module's
 * output is Y = SiLU(Conv1D(RMSNorm(V~))) + V~.  engram_gate_forward already
 * adds V~ to the residual; this call adds the remaining term in place:
 *   n_t      = V~_t / sqrt(mean_c(V~_t[c]^2) + eps) * gamma        (per token)
 *   z_t[c]   = sum_{j < taps} w[c][j] * n_{t - j*dilation}[c]      (zero before the
 *                                                                  sequence start)
 *   out_t[c] = out_t[c] + SiLU(z_t[c]),   SiLU(z) = z / (1 + e^-z)
 * so tap j looks j*dilation tokens back; the pages' configuration is taps = 4
 * and dilation = the largest n-gram order.  Sequences never mix.
 * value: device [batch * seq][d_model] (sequence-major: token t of sequence b is
 *        row b*seq + t).  out: device, same shape, updated in place; it must not
 *        overlap `value`.
 * w:     device [d_model][taps] (channel-major: the taps of one channel are
 *        contiguous).  gamma: device [d_model].  All of `dtype`, 16-byte aligned.
 * Arithmetic: fp32 for bf16 values, fp64 for fp32 values; one rounding to `dtype` when
 * `out` is written.
 * Shapes: d_model * sizeof(dtype) % 16 == 0, 1 <= taps <= ENGRAM_CONV_MAX_TAPS,
 * 1 <= dilation <= ENGRAM_CONV_MAX_DILATION, seq * d_model * sizeof(dtype) < 4 GiB
 * (UNSUPPORTED otherwise).  batch == 0
 * or seq == 0 is a no-op.  Uses the library's per-device scratch (4 bytes per
 * token), like engram_gate_forward.
 */
engram_status engram_conv_forward(const void* value, int32_t batch, int64_t seq, int32_t d_model,
                                  const void* w, const void* gamma, int32_t taps, int32_t dilation,
                                  float eps, engram_dtype dtype, void* out, hipStream_t stream);

/*
 * Prefetch from host-resident tables -- section 2.5 and Figure 2(b), section
 * 6.4: hash addresses are known before the layer runs, so the rows can be
 * fetched from host DRAM over PCIe into device memory ahead of use.
 * Same result as engram_gather, bit for bit, but host_tables[b] are pinned,
 * device-mapped host allocations (hipHostMalloc, e.g. engram_host_alloc or a
 * pinned torch tensor); the GPU reads the rows over PCIe and writes them to the
 * device buffer `staging` [n_tok][n_tables*w].  Intended for a side stream, with
 * events ordering the consumer after it.
 * Errors: INVALID_ARG if a table pointer is not a device-accessible pinned host
 * allocation; otherwise as engram_gather.
 */
engram_status engram_prefetch_host(const int32_t* idx, int64_t n_tok, int32_t n_tables,
                                   const void* const* host_tables, const int64_t* rows, int32_t w,
                                   engram_dtype dtype, void* staging, int32_t* err_count,
                                   hipStream_t stream);

/*
 * HBM cache of the hottest rows of host-resident tables -- section 2.5: n-gram
 * frequencies follow a Zipf law, so keeping the most used rows in a faster tier
 * (HBM, in front of the pinned host tables of Figure 2(b)) removes most of the
 * prefetch's PCIe traffic.  Three calls:
 *
 * engram_cache_select (host only, no GPU work): per table b, the `capacity` rows
 *   that occur most often in column b of the sample idx (host int32 [n][n_tables],
 *   e.g. the hash indices of the sequences being decoded); ties go to the smaller
 *   row, negative entries are ignored.  hot: host int32 [n_tables][capacity],
 *   padded with -1 when a column has fewer distinct rows.
 *
 * engram_cache_build: builds, on `stream`, and waits for it to finish:
 *   table:      device, [n_tables][slots] entries of two int32 {row, cache slot}
 *               (8-byte aligned; slots a power of two above capacity), an open-
 *               addressing hash table per table: the home entry of row r is the top
 *               log2(slots) bits of r * 0x9E3779B1 mod 2^32, collisions probe
 *               linearly, empty entries are {-1, -1};
 *   cache_rows: device [capacity][n_tables * w] of `dtype` (16-byte aligned): cache
 *               slot j of table b holds row hot[b][j] of host_tables[b] (zeros for -1).
 *   host_tables are pinned, device-mapped host memory, as for engram_prefetch_host.
 *   A hot row outside [0, rows[b]) is INVALID_ARG.
 *
 * engram_prefetch_host_cached: engram_prefetch_host through the cache: a (token,
 *   table) whose row is in the cache is read from cache_rows, any other from the
 *   host table over PCIe.  staging receives exactly engram_gather's result.
 *   hits: device int32 counter incremented once per cached (token, table), or NULL;
 *   err_count as for engram_gather.  slots must be the value the table was built
 *   with: the kernel reads table[b][0 .. slots-1].  A probe stops after slots entries
 *   (a smaller table than claimed then reads as misses, never loops).
 */
engram_status engram_cache_select(const int32_t* idx, int64_t n, int32_t n_tables, int32_t capacity,
                                  int32_t* hot);
engram_status engram_cache_build(const void* const* host_tables, const int64_t* rows, int32_t n_tables, int32_t w,
                                 engram_dtype dtype, const int32_t* hot, int32_t capacity, int32_t slots,
                                 void* table, void* cache_rows, hipStream_t stream);
engram_status engram_prefetch_host_cached(const int32_t* idx, int64_t n_tok, int32_t n_tables,
                                          const void* const* host_tables, const int64_t* rows, int32_t w,
                                          engram_dtype dtype, const void* table, int32_t slots,
                                          const void* cache_rows, void* staging, int32_t* hits,
                                          int32_t* err_count, hipStream_t stream);

/*
 * FP8 quantization of a row-major matrix -- section 2.4 names FP8 for the projection
 * GEMM but no format or scaling; this library's reading (the one its FP8 gate uses):
 * OCP E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa bits; 0x7E = 448 is the
 * largest finite value) with one fp32 scale per row:
 *   scales[r]     = max_c |src[r][c]| / 448   (1 for an all-zero row), in fp32
 *   codes[r][c]   = E4M3 code nearest to src[r][c] / scales[r] (the division in fp32;
 *                   ties to the even code; magnitudes >= 448 saturate to 448)
 *   sumsq[r]      = sum_c (value(codes[r][c]) * scales[r])^2 in fp32, or NULL
 * src: device [rows][cols] of dtype; codes: device uint8 [rows][cols]; scales, sumsq:
 * device float [rows].  cols % 16 == 0 (UNSUPPORTED otherwise); 16-byte aligned src
 * and codes.
 */
engram_status engram_quantize_fp8(const void* src, int64_t rows, int32_t cols, engram_dtype dtype, uint8_t* codes,
                                  float* scales, float* sumsq, hipStream_t stream);

/*
 * Context-aware gating with FP8 projections -- section 2.4 (the projections as FP8
 * matrix multiplications) applied to engram_gate_forward's computation.  The same
 * arguments and results as engram_gate_forward, with these differences:
 *   - the operands of both projections are the per-row E4M3 quantizations of
 *     engram_quantize_fp8: the key weights (with ENGRAM_KEY_NORM_MEMORY the matrix
 *     gq[m][f] * Wk[m][f][c] * gk[m][c], formed in fp32, otherwise Wk[m] itself), Wv[m],
 *     and every memory vector mem_t; k and v are the exact products of the decoded
 *     codes times the two rows' scales, accumulated in fp32;
 *   - with ENGRAM_KEY_NORM_MEMORY the memory vector's norm is that of its quantized
 *     (decoded and scaled) form;
 *   - dtype must be ENGRAM_BF16 and d_mem % 128 == 0 (UNSUPPORTED otherwise).
 * The codes are made on every call, in library-owned scratch.
 */
engram_status engram_gate_forward_fp8(const void* mem, int64_t n_tok, int32_t d_mem, int32_t d_model,
                                      int32_t n_branch, const void* const* h, const void* const* wk,
                                      const void* const* wv, const void* const* gq,
                                      const void* const* gk, float eps, engram_dtype dtype,
                                      engram_key_norm key_norm, void* const* out, float* gate_out,
                                      void* const* value_out, hipStream_t stream);

/*
 * The FP8 gate's weights, prepared once -- section 2.4.  Per branch m, the E4M3 codes
 * and per-feature scales (engram_quantize_fp8's definition) of the key weights and of
 * W_V[m], exactly as engram_gate_forward_fp8 makes them on every call: the key weights
 * are gq[m][f] * W_K[m][f][c] * gk[m][c] formed in fp32 for ENGRAM_KEY_NORM_MEMORY and
 * W_K[m] itself for ENGRAM_KEY_NORM_PROJECTED (gq, gk are then not read and may be NULL).
 * wk, wv: host arrays of n_branch device bf16 [d_model][d_mem] (16-byte aligned); gq:
 *         [d_model], gk: [d_mem] bf16.
 * wk_codes, wv_codes: host arrays of n_branch device uint8 [d_model][d_mem], 16-byte
 *         aligned; wk_scales, wv_scales: host arrays of n_branch device float [d_model].
 * d_mem % 128 == 0 and d_model % 32 == 0 (UNSUPPORTED otherwise).
 */
engram_status engram_gate_prepare_fp8(int32_t d_mem, int32_t d_model, int32_t n_branch, const void* const* wk,
                                      const void* const* wv, const void* const* gq, const void* const* gk,
                                      engram_key_norm key_norm, uint8_t* const* wk_codes, float* const* wk_scales,
                                      uint8_t* const* wv_codes, float* const* wv_scales, hipStream_t stream);

/*
 * The FP8 gate on quantized operands -- section 2.3, Eq. (3)-(4), section 2.4: the
 * results of engram_gate_forward_fp8 given the quantizations it would make itself.
 * codes, scales, sumsq: the memory vectors as engram_lookup_fp8 or engram_quantize_fp8
 *         write them ([n_tok][d_mem] uint8, 16-byte aligned; [n_tok] float); sumsq may
 *         be NULL for ENGRAM_KEY_NORM_PROJECTED.
 * wk_codes .. wv_scales: as engram_gate_prepare_fp8 writes them, with the same key_norm;
 *         branches sharing one W_V pass the same codes and scales pointers (W_V e is then
 *         computed once).
 * h, gq, gk, eps, key_norm, out, gate_out, value_out: as for engram_gate_forward (bf16;
 *         gq and gk are read for ENGRAM_KEY_NORM_PROJECTED, and must be valid pointers
 *         either way).
 * d_mem % 128 == 0 and d_model % 32 == 0 (UNSUPPORTED otherwise).
 */
engram_status engram_gate_forward_fp8q(const uint8_t* codes, const float* scales, const float* sumsq, int64_t n_tok,
                                       int32_t d_mem, int32_t d_model, int32_t n_branch, const void* const* h,
                                       const uint8_t* const* wk_codes, const float* const* wk_scales,
                                       const uint8_t* const* wv_codes, const float* const* wv_scales,
                                       const void* const* gq, const void* const* gk, float eps,
                                       engram_key_norm key_norm, void* const* out, float* gate_out,
                                       void* const* value_out, hipStream_t stream);

/* Pinned, device-mapped host allocation for offloaded tables (hipHostMalloc,
 * hipHostMallocMapped | hipHostMallocPortable). *ptr is NULL on failure. */
engram_status engram_host_alloc(size_t bytes, void** ptr);
engram_status engram_host_free(void* ptr);

#ifdef __cplusplus
}
#endif

#endif /* ENGRAM_H */
