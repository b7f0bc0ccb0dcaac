/*
 * engram_oracle.c -- plain, single-threaded CPU oracle of the Engram forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: it exists so that tests, the smoke check and the benchmark's CPU
 * baseline can compare the HIP library against an obviously correct definition.
 * It shares no code, header, table or constant with the HIP library.
 *
 * Source of the method: "Conditional Memory via Scalable Lookup: A New Axis of
 * Sparsity for Large Language Models" (DeepSeek-AI & Peking University), as
 * translated on the pages studied, and the review page "Engram: LLM에 '기억의
 * 서랍'을 달아주다" (koala.ai.kr), whose pseudocode gives the gate's order of
 * operations.  Each function names the passage it follows.
 *
 * Readings of points the pages leave open (see the design notes):
 *   - hash: z = (XOR_j  x'_{t-j} * c[n][k][j]  mod 2^64) mod M[n][k], one odd
 *     64-bit multiplier per (order, head, position in the gram); positions
 *     before the start of a sequence read the id `pad_id`;
 *   - gate: key = W_K * RMSNorm(e) (normalised before the projection; the paper's
 *     Eq. (4) placement, RMSNorm after W_K, is the key_norm = 1 mode), the scale is
 *     1/sqrt(d_model), RMSNorm(x) = x / sqrt(mean(x^2) + eps) * gamma;
 *   - short causal convolution (Eq. (5)): tap j looks j * dilation tokens back;
 *   - FP8 projections (section 2.4 names FP8 for the fused projection GEMM, without a
 *     format or a scaling): OCP E4M3, a scale per row of each operand (per token for
 *     the memory vector, per output feature for the weights) equal to max|x| / 448 in
 *     fp32, codes by round-to-nearest-even with saturation to +-448.
 *
 * Arithmetic: integers in uint64 with C's own '%' (no reduction tricks);
 * floating point decoded exactly to double, accumulated in double, sigmoid as
 * 1 / (1 + exp(-x)) in double.  Results are returned in double; callers round.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* Exact decode of one element of a float32 or bfloat16 array to double. */
static double load_elem(const void* base, int64_t i, int dtype) {
  if (dtype == ORACLE_F32) {
    return (double)((const float*)base)[i];
  }
  uint16_t b = ((const uint16_t*)base)[i];
  uint32_t u = (uint32_t)b << 16; /* bfloat16 is the top half of a float32 */
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/*
 * Tokenizer compression (section 2.2, "tokenizer compression"): each raw id is
 * replaced by its canonical id through the precomputed surjection P.
 *   out[i] = map[raw[i]]   for 0 <= raw[i] < vocab,  else -1.
 * Returns the number of out-of-range raw ids.
 */
int64_t oracle_compress(const int32_t* raw, int64_t n, const int32_t* map, int32_t vocab,
                        int32_t* out) {
  int64_t bad = 0;
  for (int64_t i = 0; i < n; ++i) {
    int32_t x = raw[i];
    if (x >= 0 && x < vocab) {
      out[i] = map[x];
    } else {
      out[i] = -1;
      ++bad;
    }
  }
  return bad;
}

/*
 * Multi-head hashing of suffix n-grams (section 2.2, Eq. (1)).
 * For every sequence b < batch, position t in [t_begin, t_begin + t_count),
 * order index o (n = orders[o]) and head k < heads:
 *   g_{t,n}   = (x'_{t-n+1}, ..., x'_t)              (suffix n-gram)
 *   h         = XOR over j = 0..n-1 of ( x'_{t-j} * mult[o][k][j]  mod 2^64 )
 *   z_{t,n,k} = h mod rows[o*heads + k]
 * x'_{t-j} for t-j < 0 is pad_id.  ids is [batch][ld] row-major; mult is
 * [n_orders][heads][max_order]; idx is [batch*t_count][n_orders*heads] with the
 * column o*heads + k (order-major, head-minor, the concatenation order of Eq. (2)).
 */
void oracle_hash(const int32_t* ids, int32_t batch, int64_t ld, int64_t t_begin, int64_t t_count,
                 const int32_t* orders, int32_t n_orders, int32_t heads, int32_t max_order,
                 const uint64_t* mult, const uint32_t* rows, int32_t pad_id, int32_t* idx) {
  const int32_t n_tables = n_orders * heads;
  for (int32_t b = 0; b < batch; ++b) {
    for (int64_t dt = 0; dt < t_count; ++dt) {
      const int64_t t = t_begin + dt;
      int32_t* row_out = idx + ((int64_t)b * t_count + dt) * n_tables;
      for (int32_t o = 0; o < n_orders; ++o) {
        const int32_t n = orders[o];
        for (int32_t k = 0; k < heads; ++k) {
          uint64_t h = 0;
          for (int32_t j = 0; j < n; ++j) {
            const int64_t pos = t - j;
            const int32_t x = pos >= 0 ? ids[(int64_t)b * ld + pos] : pad_id;
            const uint64_t c = mult[((int64_t)o * heads + k) * max_order + j];
            h ^= (uint64_t)(uint32_t)x * c; /* unsigned wrap = mod 2^64 */
          }
          const uint64_t m = rows[o * heads + k];
          row_out[o * heads + k] = (int32_t)(h % m);
        }
      }
    }
  }
}

/*
 * Table lookup and concatenation (section 2.2, Eq. (1)-(2)):
 *   e_t = concat over tables b (order-major, head-minor) of E_b[z_{t,b}].
 * tables[b] points at a row-major [rows][row_bytes] array; the copy is bitwise.
 */
void oracle_gather(const int32_t* idx, int64_t n_tok, int32_t n_tables, const void* const* tables,
                   int32_t row_bytes, void* out) {
  for (int64_t t = 0; t < n_tok; ++t) {
    for (int32_t b = 0; b < n_tables; ++b) {
      const int64_t r = idx[t * n_tables + b];
      const char* src = (const char*)tables[b] + r * (int64_t)row_bytes;
      char* dst = (char*)out + (t * n_tables + b) * (int64_t)row_bytes;
      memcpy(dst, src, (size_t)row_bytes);
    }
  }
}

/*
 * Context-aware gating of one branch (section 2.3, Eq. (3)-(4), the gated value
 * and the residual update; section 2.4, Eq. (6) for a branch m).  Two placements of
 * the key's RMSNorm:
 *   key_norm == 0 (the review page's context_aware_gating pseudocode):
 *     k = W_K * RMSNorm_{gk}(e_t),   gk: [d_mem]
 *   key_norm == 1 (the paper's Eq. (4) and Eq. (6): the key is normalised after W_K):
 *     k = RMSNorm_{gk}(W_K * e_t),   gk: [d_model]
 * and in both
 *   q     = RMSNorm_{gq}(h_t)
 *   v     = W_V * e_t
 *   alpha = sigmoid( q . k / sqrt(d_model) )
 *   out   = h_t + alpha * v
 * with RMSNorm_g(x) = x / sqrt(mean(x^2) + eps) * g.
 * mem: [n_tok][d_mem]; h, out: [n_tok][d_model]; W_K, W_V: [d_model][d_mem]
 * row-major (output x input); gq: [d_model]; all of `dtype`.
 * out and alpha are double; `value` (double [n_tok][d_model], or NULL) receives the
 * gated value alpha * v that the convolution of Eq. (5) consumes.  Returns 0, or -1
 * for an unknown key_norm.
 */
int oracle_gate(const void* mem, int64_t n_tok, int32_t d_mem, int32_t d_model, const void* h,
                const void* wk, const void* wv, const void* gq, const void* gk, double eps,
                int32_t dtype, int32_t key_norm, double* out, double* alpha, double* value) {
  if (key_norm != 0 && key_norm != 1) return -1;
  for (int64_t t = 0; t < n_tok; ++t) {
    /* RMSNorm of the memory vector and of the hidden state */
    double ss_e = 0.0;
    for (int32_t j = 0; j < d_mem; ++j) {
      const double e = load_elem(mem, t * d_mem + j, dtype);
      ss_e += e * e;
    }
    const double rms_e = sqrt(ss_e / d_mem + eps);
    double ss_h = 0.0;
    for (int32_t i = 0; i < d_model; ++i) {
      const double x = load_elem(h, t * d_model + i, dtype);
      ss_h += x * x;
    }
    const double rms_h = sqrt(ss_h / d_model + eps);

    /* logit = sum_i q_i * k_i */
    double logit = 0.0;
    if (key_norm == 0) {
      for (int32_t i = 0; i < d_model; ++i) {
        double k = 0.0;
        for (int32_t j = 0; j < d_mem; ++j) {
          const double en = load_elem(mem, t * d_mem + j, dtype) / rms_e * load_elem(gk, j, dtype);
          k += load_elem(wk, (int64_t)i * d_mem + j, dtype) * en;
        }
        const double q = load_elem(h, t * d_model + i, dtype) / rms_h * load_elem(gq, i, dtype);
        logit += q * k;
      }
    } else {
      /* the raw projection first, then its RMSNorm over the d_model features */
      double* k = (double*)malloc(sizeof(double) * (size_t)d_model);
      if (k == NULL) return -2;
      double ss_k = 0.0;
      for (int32_t i = 0; i < d_model; ++i) {
        k[i] = 0.0;
        for (int32_t j = 0; j < d_mem; ++j)
          k[i] += load_elem(wk, (int64_t)i * d_mem + j, dtype) * load_elem(mem, t * d_mem + j, dtype);
        ss_k += k[i] * k[i];
      }
      const double rms_k = sqrt(ss_k / d_model + eps);
      for (int32_t i = 0; i < d_model; ++i) {
        const double q = load_elem(h, t * d_model + i, dtype) / rms_h * load_elem(gq, i, dtype);
        logit += q * (k[i] / rms_k * load_elem(gk, i, dtype));
      }
      free(k);
    }
    logit /= sqrt((double)d_model);
    const double a = 1.0 / (1.0 + exp(-logit));
    alpha[t] = a;

    /* value projection and residual update */
    for (int32_t i = 0; i < d_model; ++i) {
      double v = 0.0;
      for (int32_t j = 0; j < d_mem; ++j) {
        v += load_elem(wv, (int64_t)i * d_mem + j, dtype) * load_elem(mem, t * d_mem + j, dtype);
      }
      out[t * d_model + i] = load_elem(h, t * d_model + i, dtype) + a * v;
      if (value != NULL) value[t * d_model + i] = a * v;
    }
  }
  return 0;
}

/*
 * Short depthwise causal convolution over the gated values (section 2.3, Eq. (5)).
 * With V~ the sequence of gated values of one sequence (token t, channel c):
 *   n_t     = RMSNorm_{gamma}(V~_t)            = V~_t / sqrt(mean_c(V~_t^2) + eps) * gamma
 *   z_{t,c} = sum_{j=0}^{taps-1} w[c][j] * n_{t - j*dil, c}    (zero before the sequence start)
 *   Y_t     = SiLU(z_t) + V~_t,    SiLU(x) = x / (1 + exp(-x))
 * and the layer output is h_t + Y_t.  `base` holds h_t + V~_t (what the gate writes), so
 *   out = base + SiLU(z).
 * Tap j reads the token j*dil positions back (the kernel covers lags 0, dil, ..,
 * (taps-1)*dil).  value, base, out: double [batch*seq][d_model] (token b*seq + t);
 * w: [d_model][taps] and gamma: [d_model] of `dtype`.
 */
void oracle_conv(const double* value, int32_t batch, int64_t seq, int32_t d_model, const void* w,
                 const void* gamma, int32_t taps, int32_t dil, double eps, int32_t dtype,
                 const double* base, double* out) {
  const int64_t n_tok = (int64_t)batch * seq;
  for (int64_t t = 0; t < n_tok; ++t) {
    for (int32_t c = 0; c < d_model; ++c) out[t * d_model + c] = base[t * d_model + c];
  }
  for (int32_t b = 0; b < batch; ++b) {
    for (int64_t t = 0; t < seq; ++t) {
      for (int32_t c = 0; c < d_model; ++c) {
        double z = 0.0;
        for (int32_t j = 0; j < taps; ++j) {
          const int64_t ts = t - (int64_t)j * dil;
          if (ts < 0) continue;
          const double* row = value + ((int64_t)b * seq + ts) * d_model;
          double ss = 0.0;
          for (int32_t k = 0; k < d_model; ++k) ss += row[k] * row[k];
          const double n = row[c] / sqrt(ss / d_model + eps) * load_elem(gamma, c, dtype);
          z += load_elem(w, (int64_t)c * taps + j, dtype) * n;
        }
        out[((int64_t)b * seq + t) * d_model + c] += z / (1.0 + exp(-z));
      }
    }
  }
}

/*
 * FP8 E4M3 (the OCP 8-bit floating point format, E4M3 variant): 1 sign bit, 4 exponent
 * bits with bias 7, 3 mantissa bits.  Exponent field 0 holds the subnormals m * 2^-9;
 * field e > 0 the normals (1 + m/8) * 2^(e-7); 0x7F and 0xFF are NaN, so the largest
 * finite magnitude is 0x7E = 1.75 * 2^8 = 448.  No infinities.
 */
double oracle_e4m3_decode(uint8_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp(1.0 + m / 8.0, e - 7);
  return (c & 0x80) ? -v : v;
}

/* The code nearest to v (ties to the even code), magnitudes of 448 and above saturate
 * to 448.  Works on the exact value of v in double: the representable magnitudes in
 * [2^E, 2^(E+1)) are spaced 2^(E-3) for E >= -6 and 2^-9 below (the subnormals). */
uint8_t oracle_e4m3_encode(float v) {
  const uint8_t sign = signbit(v) ? 0x80 : 0;
  const double a = fabs((double)v);
  if (a >= 448.0) return sign | 0x7E;
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);            /* a = f * 2^e2, f in [0.5, 1): a in [2^(e2-1), 2^e2) */
  const int E = e2 - 1;
  const double quantum = E < -6 ? ldexp(1.0, -9) : ldexp(1.0, E - 3);
  double q = a / quantum;   /* exact: a power-of-two division */
  double r = floor(q);
  const double frac = q - r;
  if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  const double val = r * quantum;
  if (val == 0.0) return sign;
  if (val >= 448.0) return sign | 0x7E;
  int f2;
  frexp(val, &f2);
  const int E2 = f2 - 1;
  if (E2 < -6) return sign | (uint8_t)(val / ldexp(1.0, -9));            /* subnormal */
  const int mant = (int)(val / ldexp(1.0, E2 - 3)) - 8;                    /* 0..7 */
  return sign | (uint8_t)(((E2 + 7) << 3) | mant);
}

/* Per row r of x [rows][cols] (float): s = max|x[r][:]| / 448 in fp32 (1 for an all-zero
 * row), codes[r][c] = encode(x[r][c] / s) with the division in fp32. */
void oracle_quant_rows(const float* x, int64_t rows, int32_t cols, uint8_t* codes, float* scales) {
  for (int64_t r = 0; r < rows; ++r) {
    const float* xr = x + r * cols;
    float mx = 0.f;
    for (int32_t c = 0; c < cols; ++c) mx = fmaxf(mx, fabsf(xr[c]));
    const float s = mx > 0.f ? mx / 448.0f : 1.0f;
    scales[r] = s;
    for (int32_t c = 0; c < cols; ++c) codes[r * cols + c] = oracle_e4m3_encode(xr[c] / s);
  }
}

/*
 * The gate of oracle_gate with its two projections in FP8 (the reading in the header):
 *   e          quantized per token:              e^  = s_e[t]  * code_e
 *   key weights: key_norm 0: W'' = (gq[f] * W_K[f][c]) * gk[c] in fp32, quantized per
 *              row f; key_norm 1: W_K quantized per row
 *   W_V        quantized per row
 * then, in double from the dequantized values,
 *   key_norm 0:  k_f = (W''^ e^)_f / rms(e^)          q_f = h_f / rms(h)
 *   key_norm 1:  k_f = (W_K^ e^)_f / rms(W_K^ e^) * gk[f],  q_f = h_f / rms(h) * gq[f]
 *   alpha = sigmoid(q . k / sqrt(d_model)),   out = h + alpha * (W_V^ e^)
 * Inputs as for oracle_gate (bf16 or f32); returns 0, or -1/-2 for a bad mode/alloc.
 */
int oracle_gate_fp8(const void* mem, int64_t n_tok, int32_t d_mem, int32_t d_model, const void* h,
                    const void* wk, const void* wv, const void* gq, const void* gk, double eps, int32_t dtype,
                    int32_t key_norm, double* out, double* alpha) {
  if (key_norm != 0 && key_norm != 1) return -1;
  const size_t nw = (size_t)d_model * d_mem;
  float* wf = (float*)malloc(sizeof(float) * nw);
  float* ef = (float*)malloc(sizeof(float) * (size_t)d_mem);
  uint8_t* ck = (uint8_t*)malloc(nw);
  uint8_t* cv = (uint8_t*)malloc(nw);
  uint8_t* ce = (uint8_t*)malloc((size_t)d_mem);
  float* sk = (float*)malloc(sizeof(float) * (size_t)d_model);
  float* sv = (float*)malloc(sizeof(float) * (size_t)d_model);
  double* k = (double*)malloc(sizeof(double) * (size_t)d_model);
  if (!wf || !ef || !ck || !cv || !ce || !sk || !sv || !k) {
    free(wf); free(ef); free(ck); free(cv); free(ce); free(sk); free(sv); free(k);
    return -2;
  }
  /* key weights */
  for (int32_t f = 0; f < d_model; ++f)
    for (int32_t c = 0; c < d_mem; ++c) {
      const float w = (float)load_elem(wk, (int64_t)f * d_mem + c, dtype);
      wf[(size_t)f * d_mem + c] =
          key_norm == 0 ? ((float)load_elem(gq, f, dtype) * w) * (float)load_elem(gk, c, dtype) : w;
    }
  oracle_quant_rows(wf, d_model, d_mem, ck, sk);
  for (size_t i = 0; i < nw; ++i) wf[i] = (float)load_elem(wv, (int64_t)i, dtype);
  oracle_quant_rows(wf, d_model, d_mem, cv, sv);
  for (int64_t t = 0; t < n_tok; ++t) {
    for (int32_t c = 0; c < d_mem; ++c) ef[c] = (float)load_elem(mem, t * d_mem + c, dtype);
    float se;
    oracle_quant_rows(ef, 1, d_mem, ce, &se);
    double ss_e = 0.0;
    for (int32_t c = 0; c < d_mem; ++c) {
      const double x = se * oracle_e4m3_decode(ce[c]);
      ss_e += x * x;
    }
    double ss_h = 0.0;
    for (int32_t i = 0; i < d_model; ++i) {
      const double x = load_elem(h, t * d_model + i, dtype);
      ss_h += x * x;
    }
    const double rms_h = sqrt(ss_h / d_model + eps);
    double ss_k = 0.0;
    for (int32_t f = 0; f < d_model; ++f) {
      double acc = 0.0;
      for (int32_t c = 0; c < d_mem; ++c)
        acc += oracle_e4m3_decode(ck[(size_t)f * d_mem + c]) * oracle_e4m3_decode(ce[c]);
      k[f] = (double)sk[f] * se * acc;
      ss_k += k[f] * k[f];
    }
    double logit = 0.0;
    if (key_norm == 0) {
      const double rms_e = sqrt(ss_e / d_mem + eps);
      for (int32_t f = 0; f < d_model; ++f) logit += load_elem(h, t * d_model + f, dtype) / rms_h * (k[f] / rms_e);
    } else {
      const double rms_k = sqrt(ss_k / d_model + eps);
      for (int32_t f = 0; f < d_model; ++f)
        logit += load_elem(h, t * d_model + f, dtype) / rms_h * load_elem(gq, f, dtype) *
                 (k[f] / rms_k * load_elem(gk, f, dtype));
    }
    logit /= sqrt((double)d_model);
    const double a = 1.0 / (1.0 + exp(-logit));
    alpha[t] = a;
    for (int32_t f = 0; f < d_model; ++f) {
      double acc = 0.0;
      for (int32_t c = 0; c < d_mem; ++c)
        acc += oracle_e4m3_decode(cv[(size_t)f * d_mem + c]) * oracle_e4m3_decode(ce[c]);
      out[t * d_model + f] = load_elem(h, t * d_model + f, dtype) + a * ((double)sv[f] * se * acc);
    }
  }
  free(wf); free(ef); free(ck); free(cv); free(ce); free(sk); free(sv); free(k);
  return 0;
}
