// hash.hip -- multi-head multiply-XOR hashing of suffix n-grams.
// "Conditional Memory via Scalable Lookup", section 2.2, Eq. (1): for each
// position t, n-gram order n and head k, the suffix n-gram of canonical ids is
// mapped by its own hash function into a prime-sized table.  The hash is the
// lightweight multiply-XOR form:
//   h = XOR_j ( x'_{t-j} * c[n][k][j] mod 2^64 ),   z = h mod M[n][k].
//
// Layout of the work: one thread per (position, table) pair, table index
// fastest, so a wavefront writes consecutive int32 entries of the token-major
// index matrix [tokens][tables].  A workgroup owns POS consecutive positions of
// one sequence and first stages their ids plus the (max_order - 1) ids before
// them in LDS; every thread then reads its n ids from LDS.  engram_compress_hash
// reads raw ids instead and maps them through the compression table as it stages
// them, which saves the compress kernel's launch and its pass over the ids.
//
// The 64-bit reduction modulo a prime M < 2^31 uses a Barrett quotient with the
// host-computed constant m = floor((2^64 - 1) / M):  q = mulhi(h, m) is either
// floor(h / M) or one less, so r = h - q * M needs at most one subtraction.
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int POS = 64;  // positions per workgroup

__global__ __launch_bounds__(256) void hash_kernel(const HashArgs a) {
  __shared__ int32_t s_ids[POS + ENGRAM_MAX_ORDER - 1];
  const uint32_t nblk = (uint32_t)((a.t_count + POS - 1) / POS);  // workgroups per sequence
  const int32_t b = (int32_t)(blockIdx.x / nblk);
  const int64_t p0 = (int64_t)(blockIdx.x - (uint32_t)b * nblk) * POS;  // window-relative start
  const int64_t t0 = a.t_begin + p0;                       // absolute first position
  const int halo = a.max_order - 1;
  const int64_t npos = (a.t_count - p0) < POS ? (a.t_count - p0) : POS;
  const int32_t* row = a.ids + (int64_t)b * a.ld;

  int bad = 0;
  for (int i = threadIdx.x; i < npos + halo; i += blockDim.x) {
    const int64_t t = t0 - halo + i;
    int32_t x = a.pad_id;
    if (t >= 0) {
      x = row[t];
      if (a.map != nullptr) {  // tokenizer compression on the way in (section 2.2)
        const bool ok = (uint32_t)x < (uint32_t)a.vocab;
        x = ok ? a.map[x] : -1;
        if (i >= halo) {  // positions of this workgroup's window: write and count once
          if (a.ids_out != nullptr) a.ids_out[(int64_t)b * a.ld + t] = x;
          bad += ok ? 0 : 1;
        }
      }
    }
    s_ids[i] = x;
  }
  if (a.err_count != nullptr) {
    for (int off = 32; off > 0; off >>= 1) bad += __shfl_xor(bad, off, 64);
    if ((threadIdx.x & 63) == 0 && bad != 0) atomicAdd(a.err_count, bad);
  }
  __syncthreads();

  const int nt = a.n_tables;
  int32_t* out = a.idx + ((int64_t)b * a.t_count + p0) * nt;
  const int pairs = (int)npos * nt;
  for (int q = threadIdx.x; q < pairs; q += blockDim.x) {
    const int pos = q / nt;
    const int tb = q - pos * nt;
    const int n = a.order[tb];
    const int32_t* g = s_ids + pos + halo;  // g[-j] is x'_{t-j}
    uint64_t h = 0;
    for (int j = 0; j < n; ++j) h ^= (uint64_t)(uint32_t)g[-j] * a.mult[tb][j];
    out[q] = (int32_t)mod_barrett(h, a.rows[tb], a.barrett[tb]);
  }
}

// For the gate that gathers its own rows: per position of the window, its canonical id
// and the three before it (the pad id before the sequence's start), one int4 per
// position.  Raw ids are mapped as the hash kernel maps them, and each window position's
// own id is written to ids_out and counted (once) there too.
__global__ __launch_bounds__(256) void gate_ids_kernel(const HashArgs a, int4* ids) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= (int64_t)a.batch * a.t_count) return;
  const int64_t b = p / a.t_count;
  const int64_t t = a.t_begin + (p - b * a.t_count);
  const int32_t* row = a.ids + b * a.ld;
  int32_t x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = a.pad_id;
    if (t - j >= 0) {
      int32_t v = row[t - j];
      if (a.map != nullptr) {
        const bool ok = (uint32_t)v < (uint32_t)a.vocab;
        v = ok ? a.map[v] : -1;
        if (j == 0) {
          if (a.ids_out != nullptr) a.ids_out[b * a.ld + t] = v;
          if (!ok && a.err_count != nullptr) atomicAdd(a.err_count, 1);
        }
      }
      x[j] = v;
    }
  }
  ids[p] = make_int4(x[0], x[1], x[2], x[3]);
}

}  // namespace

void launch_gate_ids(const HashArgs& a, int4* ids, hipStream_t s) {
  const int64_t n = (int64_t)a.batch * a.t_count;
  hipLaunchKernelGGL(gate_ids_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, ids);
}

void launch_hash(const HashArgs& a, hipStream_t s) {
  const uint64_t nblk = (uint64_t)((a.t_count + POS - 1) / POS);
  hipLaunchKernelGGL(hash_kernel, dim3((unsigned)(nblk * (uint64_t)a.batch)), dim3(256), 0, s, a);
}

}  // namespace engram
