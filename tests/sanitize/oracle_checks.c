/* The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer: every
 * function runs on small inputs (with one known value each, from the hand-worked
 * fixtures under tests/golden/) so that an out-of-bounds access, a leak or undefined
 * behaviour in the oracle aborts the run.  Exits non-zero on a wrong value. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t oracle_compress(const int32_t* raw, int64_t n, const int32_t* map, int32_t vocab, int32_t* out);
void oracle_hash(const int32_t* ids, int32_t batch, int64_t ld, int64_t t_begin, int64_t t_count,
                 const int32_t* orders, int32_t n_orders, int32_t heads, int32_t max_order, const uint64_t* mult,
                 const uint32_t* rows, int32_t pad_id, int32_t* idx);
void oracle_gather(const int32_t* idx, int64_t n_tok, int32_t n_tables, const void* const* tables,
                   int32_t row_bytes, void* out);
int oracle_gate(const void* mem, int64_t n_tok, int32_t d_mem, int32_t d_model, const void* h, const void* wk,
                const void* wv, const void* gq, const void* gk, double eps, int32_t dtype, int32_t key_norm,
                double* out, double* alpha, double* value);
void oracle_conv(const double* value, int32_t batch, int64_t seq, int32_t d_model, const void* w,
                 const void* gamma, int32_t taps, int32_t dil, double eps, int32_t dtype, const double* base,
                 double* out);
double oracle_e4m3_decode(uint8_t c);
uint8_t oracle_e4m3_encode(float v);
void oracle_quant_rows(const float* x, int64_t rows, int32_t cols, uint8_t* codes, float* scales);
int oracle_gate_fp8(const void* mem, int64_t n_tok, int32_t d_mem, int32_t d_model, const void* h, const void* wk,
                    const void* wv, const void* gq, const void* gk, double eps, int32_t dtype, int32_t key_norm,
                    double* out, double* alpha);

static int fails = 0;
#define EXPECT(c)                                                 \
  do {                                                            \
    if (!(c)) {                                                   \
      fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #c); \
      fails++;                                                    \
    }                                                             \
  } while (0)

int main(void) {
  /* compress: one out-of-range id */
  const int32_t map[5] = {4, 3, 2, 1, 0};
  const int32_t raw[6] = {0, 5, 1, -1, 4, 2};
  int32_t ids[6];
  EXPECT(oracle_compress(raw, 6, map, 5, ids) == 2 && ids[0] == 4 && ids[1] == -1 && ids[4] == 0);

  /* hash: the worked bigram (5, 7) of tests/golden/hash_worked.txt, head (2, 0), M = 4093 */
  const int32_t seq[2] = {5, 7}, orders[2] = {2, 3};
  const uint64_t mult[2 * 2 * 3] = {0x910a2dec89025cc1ull, 0xbeeb8da1658eec67ull, 0,
                                    0xf893a2eefb32555full, 0x71c18690ee42c90bull, 0,
                                    0x71bb54d8d101b5b9ull, 0xc34d0bff90150281ull, 0xe099ec6cd7363ca5ull,
                                    0x85e7bb0f12278575ull, 0x491718de357e3da9ull, 0xcb435c8e74616797ull};
  const uint32_t rows[4] = {4093, 4093, 4093, 4093};
  int32_t idx[2 * 4];
  oracle_hash(seq, 1, 2, 0, 2, orders, 2, 2, 3, mult, rows, 770, idx);
  EXPECT(idx[4 + 0] == 1172);
  for (int i = 0; i < 8; ++i) EXPECT(idx[i] >= 0 && idx[i] < 4093);

  /* gather: concatenation order */
  float t0[3 * 4], t1[3 * 4], e[2 * 8];
  for (int i = 0; i < 12; ++i) { t0[i] = (float)i; t1[i] = (float)(100 + i); }
  const void* tabs[2] = {t0, t1};
  const int32_t gidx[4] = {2, 0, 1, 2};
  oracle_gather(gidx, 2, 2, tabs, 16, e);
  EXPECT(e[0] == 8.f && e[4] == 100.f && e[8] == 4.f && e[15] == 111.f);

  /* gate: example A of tests/golden/gate_micro.txt, both key placements, with values */
  const float me[2] = {0.3f, -0.4f}, h[2] = {1.f, 2.f}, wk[4] = {2, 1, 0, 1}, wv[4] = {2, 0, 1, 1};
  const float one[2] = {1.f, 1.f};
  double out[2], alpha[1], val[2];
  EXPECT(oracle_gate(me, 1, 2, 2, h, wk, wv, one, one, 0.0, 0, 0, out, alpha, val) == 0);
  EXPECT(fabs(alpha[0] - 0.318875) < 1e-6 && fabs(out[0] - 1.191325) < 1e-6 && fabs(val[1] - (out[1] - 2)) < 1e-12);
  EXPECT(oracle_gate(me, 1, 2, 2, h, wk, wv, one, one, 0.0, 0, 1, out, alpha, NULL) == 0);
  EXPECT(oracle_gate(me, 1, 2, 2, h, wk, wv, one, one, 0.0, 0, 2, out, alpha, NULL) == -1);

  /* FP8: example E (exact in E4M3), and codes round-trip */
  const float e_E[2] = {0.5f, -0.25f}, h_E[2] = {1.f, -2.f}, wk_E[4] = {1.f, -0.5f, 0.25f, -1.f};
  const float wv_E[4] = {1.f, 1.f, 0.5f, -2.f}, gq_E[2] = {2.f, 0.5f}, gk_E[2] = {0.5f, 2.f};
  EXPECT(oracle_gate_fp8(e_E, 1, 2, 2, h_E, wk_E, wv_E, gq_E, gk_E, 0.0, 0, 0, out, alpha) == 0);
  EXPECT(fabs(alpha[0] - 0.621277653347326) < 1e-6);  /* the scales are fp32 quotients */
  for (int c = 0; c < 256; ++c)
    if ((c & 0x7f) != 0x7f) EXPECT(oracle_e4m3_encode((float)oracle_e4m3_decode((uint8_t)c)) == (uint8_t)c || (c == 0x80));
  float x[2 * 16];
  uint8_t codes[2 * 16];
  float sc[2];
  for (int i = 0; i < 32; ++i) x[i] = (float)(i - 11) * 0.37f;
  oracle_quant_rows(x, 2, 16, codes, sc);
  EXPECT(fabs(oracle_e4m3_decode(codes[0]) * sc[0] - x[0]) <= fabs(x[0]) / 16);

  /* convolution: a zero kernel leaves the base */
  double v[2 * 5 * 3], base[2 * 5 * 3], co[2 * 5 * 3];
  for (int i = 0; i < 30; ++i) { v[i] = sin(i); base[i] = cos(i); }
  const float w0[3 * 4] = {0}, g3[3] = {1.f, 2.f, 0.5f};
  oracle_conv(v, 2, 5, 3, w0, g3, 4, 3, 1e-6, 0, base, co);
  EXPECT(memcmp(co, base, sizeof co) == 0);
  const float w1[3 * 4] = {1, -1, 2, 0.5, 0.5, 0.25, -2, 1, -1, 1.5, 0.75, -0.5};
  oracle_conv(v, 2, 5, 3, w1, g3, 4, 3, 1e-6, 0, base, co);
  for (int i = 0; i < 30; ++i) EXPECT(isfinite(co[i]));

  if (fails) return 1;
  printf("oracle checks passed\n");
  return 0;
}
