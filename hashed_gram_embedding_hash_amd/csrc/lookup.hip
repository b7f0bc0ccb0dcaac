// lookup.hip -- compression, hashing and the row gather in one kernel.
// "Conditional Memory via Scalable Lookup", section 2.2, Eq. (1)-(2): map each raw id
// to its canonical id, hash every suffix n-gram of every position into its tables,
// and concatenate the selected rows into the position's memory vector.  The results
// are those of engram_compress_hash followed by engram_gather, bit for bit; the
// indices never leave LDS unless the caller asks for them.
//
// A workgroup owns P = ty * U consecutive positions of one sequence:
//   1. it stages their ids and the (max_order - 1) before them in LDS (through the
//      compression map when one is given), as the hash kernel does;
//   2. one thread per (position, table) computes the index into LDS;
//   3. the gather kernel's layout: threadIdx.x is the 16-byte chunk of the
//      concatenated row, threadIdx.y the position, U positions per thread with all
//      U loads issued before the stores; the workgroup's output is one contiguous
//      span of P rows.
// The first two steps cost one dependent round trip for the ids; they replace a
// launch, its tail and the index matrix's write and read.
//
// engram_lookup_fp8 (Q8): bf16 rows, and instead of storing them each position's
// memory vector is quantized as engram_quantize_fp8 does (section 2.4): its maximum
// magnitude is reduced across the row's lanes in LDS (an integer max of the float
// bits: order-free), every lane encodes its 8 values against the row's scale, and
// the row's sum of squares of the dequantized values is summed in a fixed order (the
// result does not depend on timing).
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int LK_U = 8;          // positions per thread in the gather step
constexpr int LK_MAX_P = 64;     // positions per workgroup, at most

template <int U, bool Q8>
__global__ __launch_bounds__(1024) void lookup_kernel(const HashArgs h, const GatherArgs g, const Q8Out q) {
  // dynamic LDS: the P positions' indices, then their ids with the halo; Q8 adds the
  // rows' maxima and the lanes' partial sums of squares
  extern __shared__ int32_t lk_smem[];
  const int cpt = blockDim.x;                     // 16-byte chunks per output row
  const int tid = threadIdx.y * cpt + threadIdx.x;
  const int nthr = cpt * blockDim.y;
  const int P = blockDim.y * U;
  int32_t* s_idx = lk_smem;                       // [P][n_tables]
  int32_t* s_ids = lk_smem + P * h.n_tables;      // [P + max_order - 1]
  const uint32_t nblk = (uint32_t)((h.t_count + P - 1) / P);  // workgroups per sequence
  const int32_t b = (int32_t)(blockIdx.x / nblk);
  const int64_t p0 = (int64_t)(blockIdx.x - (uint32_t)b * nblk) * P;  // window-relative start
  const int64_t t0 = h.t_begin + p0;
  const int halo = h.max_order - 1;
  const int npos = (int)((h.t_count - p0) < P ? (h.t_count - p0) : P);
  const int32_t* row = h.ids + (int64_t)b * h.ld;

  uint32_t* s_max = reinterpret_cast<uint32_t*>(s_ids + P + ENGRAM_MAX_ORDER - 1);  // Q8: [P]
  float* s_part = reinterpret_cast<float*>(s_max + P);                               // Q8: [P][cpt]
  if constexpr (Q8) {
    for (int i = tid; i < P; i += nthr) s_max[i] = 0u;  // published by the barrier below
  }

  // 1. ids, mapped on the way in
  for (int i = tid; i < npos + halo; i += nthr) {
    const int64_t t = t0 - halo + i;
    int32_t x = h.pad_id;
    if (t >= 0) {
      x = row[t];
      if (h.map != nullptr) {
        const bool ok = (uint32_t)x < (uint32_t)h.vocab;
        x = ok ? h.map[x] : -1;
        if (i >= halo) {  // this workgroup's own positions: write and count once
          if (h.ids_out != nullptr) h.ids_out[(int64_t)b * h.ld + t] = x;
          if (!ok && h.err_count != nullptr) atomicAdd(h.err_count, 1);
        }
      }
    }
    s_ids[i] = x;
  }
  __syncthreads();

  // 2. indices
  const int nt = h.n_tables;
  int32_t* idx_out = h.idx != nullptr ? h.idx + ((int64_t)b * h.t_count + p0) * nt : nullptr;
  for (int q = tid; q < npos * nt; q += nthr) {
    const int pos = q / nt;
    const int tb = q - pos * nt;
    const int n = h.order[tb];
    const int32_t* gr = s_ids + pos + halo;  // gr[-j] is x'_{t-j}
    uint64_t hv = 0;
    for (int j = 0; j < n; ++j) hv ^= (uint64_t)(uint32_t)gr[-j] * h.mult[tb][j];
    const int32_t z = (int32_t)mod_barrett(hv, h.rows[tb], h.barrett[tb]);
    s_idx[q] = z;
    if (idx_out != nullptr) idx_out[q] = z;
  }
  __syncthreads();

  // 3. rows
  const int c = threadIdx.x;
  const int cpr = g.chunks_per_row;
  const int tb = c / cpr;
  const int k = c - tb * cpr;
  const char* tab = g.table[tb];
  const int64_t row_bytes = (int64_t)cpr * 16;
  char* out = g.out + ((int64_t)b * h.t_count + p0) * (row_bytes * nt);
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int pos = threadIdx.y + u * blockDim.y;
    v[u] = make_uint4(0u, 0u, 0u, 0u);
    if (pos < npos) v[u] = *reinterpret_cast<const uint4*>(tab + (int64_t)s_idx[pos * nt + tb] * row_bytes + k * 16);
  }
  if constexpr (!Q8) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pos = threadIdx.y + u * blockDim.y;
      if (pos < npos) *reinterpret_cast<uint4*>(out + (int64_t)pos * (row_bytes * nt) + c * 16) = v[u];
    }
  } else {
    // 4. quantize: the row maximum, then the codes and the partial sums of squares
    auto bf = [](uint32_t w, bool hi) { return __uint_as_float(hi ? (w & 0xffff0000u) : (w << 16)); };
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pos = threadIdx.y + u * blockDim.y;
      if (pos < npos) {
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(bf(w[i >> 1], i & 1)));
        atomicMax(s_max + pos, __float_as_uint(m));  // non-negative floats order as integers
      }
    }
    __syncthreads();
    const int d_mem = cpt * 8;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pos = threadIdx.y + u * blockDim.y;
      if (pos < npos) {
        const float mx = __uint_as_float(s_max[pos]);
        const float sc = mx > 0.f ? mx / 448.0f : 1.0f;
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        const uint32_t c0 = e4m3_pack4(bf(w[0], false) / sc, bf(w[0], true) / sc, bf(w[1], false) / sc, bf(w[1], true) / sc);
        const uint32_t c1 = e4m3_pack4(bf(w[2], false) / sc, bf(w[2], true) / sc, bf(w[3], false) / sc, bf(w[3], true) / sc);
        const int64_t row = (int64_t)b * h.t_count + p0 + pos;
        *reinterpret_cast<uint2*>(q.codes + row * d_mem + c * 8) = make_uint2(c0, c1);
        s_part[pos * cpt + c] = sumsq4(c0, sc) + sumsq4(c1, sc);
      }
    }
    __syncthreads();
    for (int pos = tid; pos < npos; pos += nthr) {
      float ss = 0.f;
      for (int k2 = 0; k2 < cpt; ++k2) ss += s_part[pos * cpt + k2];
      const float mx = __uint_as_float(s_max[pos]);
      const int64_t row = (int64_t)b * h.t_count + p0 + pos;
      q.scales[row] = mx > 0.f ? mx / 448.0f : 1.0f;
      if (q.sumsq != nullptr) q.sumsq[row] = ss;
    }
  }
}

}  // namespace

void launch_lookup(const HashArgs& h, const GatherArgs& g, const Q8Out* q8, hipStream_t s) {
  const int cpt = g.n_tables * g.chunks_per_row;  // <= 1024, checked by the caller
  int ty = 256 / cpt;
  if (ty < 1) ty = 1;
  if (ty * LK_U > LK_MAX_P) ty = LK_MAX_P / LK_U;
  const int P = ty * LK_U;
  const uint64_t nblk = (uint64_t)((h.t_count + P - 1) / P);
  size_t lds = (size_t)(P * h.n_tables + P + ENGRAM_MAX_ORDER - 1) * sizeof(int32_t);
  const dim3 grid((unsigned)(nblk * (uint64_t)h.batch)), block(cpt, ty);
  if (q8 == nullptr) {
    hipLaunchKernelGGL((lookup_kernel<LK_U, false>), grid, block, lds, s, h, g, Q8Out{});
  } else {
    lds += (size_t)P * sizeof(uint32_t) + (size_t)P * cpt * sizeof(float);
    hipLaunchKernelGGL((lookup_kernel<LK_U, true>), grid, block, lds, s, h, g, *q8);
  }
}

}  // namespace engram
