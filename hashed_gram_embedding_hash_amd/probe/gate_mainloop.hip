// gate_mainloop.hip -- measurement probes for the benchmark, not part of the method's path:
// what bounds the bf16 gate's main loop on gfx950.
//
//   engram_probe_mainloop: the gate's k-step alone, with its shapes -- a 256 x 256 output
//     tile, 64-deep k-steps over a ring of five 32-KB LDS slots, the refill of two slots per
//     k-step spread through the MFMA stream as direct global->LDS loads, fragment reads spread
//     one per two MFMAs, one LDS barrier per k-step -- over 20-k-step tiles of synthetic bf16
//     operands, with no epilogue.  `mode` switches parts off to see which one sets the pace:
//     bit 0 no operand loads in the steady k-steps, bit 1 no fragment reads (the MFMAs reuse
//     the registers), bit 2 no MFMAs.  Four waves (2 x 2, 128 x 128 outputs each) as in the
//     gate, or eight (2 x 4, 128 x 64 each, two waves per SIMD).
//   engram_probe_mainloop_fp8: the FP8 gate's k-step the same way (four waves): a 128-byte
//     ring row holds 128 E4M3 values, each k-step is two halves of 64, each half 16
//     v_mfma_scale_f32_32x32x64_f8f6f4 per wave (2,048 cycles of matrix-core issue per
//     k-step, as in bf16) with the next half's fragments (two 16-byte reads each) read
//     one per MFMA and the refill loads one per two MFMAs.  The operand bytes stream as in
//     the bf16 probe (the values' bits are not meaningful as E4M3; timing only).
//   engram_probe_mfma: back-to-back MFMAs (16 independent accumulators, 4 x 4 distinct operand
//     registers as in a 128 x 128 wave tile), one wave per SIMD: kind 0 the bf16 gate's
//     v_mfma_f32_32x32x16_bf16, kind 1 the FP8 gate's v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3
//     operands, unit block scales).
//
// Both record, per workgroup, the shader-clock counter (s_memtime) and the constant 100-MHz
// counter (s_memrealtime) around the work, so the clock the chip actually ran at and the
// cycles per k-step or per MFMA follow.  Ordinary kernels on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int BK = 64, NSLOT = 5, SLOT_BYTES = 256 * BK * 2;
constexpr int D_MEM = 1280, NK = D_MEM / BK;  // 20 k-steps per tile, as in the large workload

__device__ __forceinline__ int row_key(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ void dma16(const uint16_t* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Tiles: workgroup b (XCD b % 8, slot w = b / 8 of 32) takes in round r the token tile
// 4 ((r / 2) 8 + b % 8) + w % 4 and the feature tile 8 (r % 2) + w / 4, so the 32 workgroups
// of an XCD share each memory tile 8 ways and each weight panel 4 ways, as in the gate.
// W: [16 * 256][D_MEM] bf16; E: [(rounds / 2) * 32 * 256 + 1024][D_MEM] bf16 (the caller
// sizes it; see engram_probe_mainloop).
template <int NW, int MODE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void probe_mainloop_kernel(const uint16_t* __restrict__ W, const uint16_t* __restrict__ E, int rounds,
                           float* __restrict__ sink, uint64_t* __restrict__ clk) {
  constexpr int WT = NW == 4 ? 128 : 64, WF = 128;
  constexpr int MF = WF / 32, MT = WT / 32, NTW = 256 / WT;
  constexpr int G = SLOT_BYTES / 1024 / NW;  // 1-KB loads per wave per slot
  __shared__ __attribute__((aligned(16))) char smem[NSLOT * SLOT_BYTES];
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf = wave / NTW, wt = wave % NTW;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr)smem;
  const uint32_t wave_dst = lds0 + (uint32_t)(wave * G * 1024);
  const int x = blockIdx.x % 8, w = blockIdx.x / 8;
  const int khalf = lane >> 5;
  const int arow0 = wf * WF + (lane & 31), brow0 = wt * WT + (lane & 31);
  uint32_t fr_a[4], fr_b[4];
#pragma unroll
  for (int ss = 0; ss < 4; ++ss) {
    fr_a[ss] = (uint32_t)(arow0 * (BK * 2) + (((ss * 2 + khalf) ^ row_key(arow0)) * 16));
    fr_b[ss] = (uint32_t)(brow0 * (BK * 2) + (((ss * 2 + khalf) ^ row_key(brow0)) * 16));
  }
  float total = 0.f;
  for (int r = 0; r < rounds; ++r) {
    const int ttile = ((r / 2) * 8 + x) * 4 + (w & 3), ftile = (r % 2) * 8 + (w >> 2);
    const uint16_t* Wt = W + (int64_t)ftile * 256 * D_MEM;
    const uint16_t* Et = E + (int64_t)ttile * 256 * D_MEM;
    uint32_t off[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int rr = wave * (G * 8) + i * 8 + (lane >> 3);
      off[i] = (uint32_t)rr * D_MEM + (((lane & 7) ^ row_key(rr)) * 8);
    }
    lds_barrier();  // the previous tile's fragment reads are done before the ring refills
    // chunk c: weight rows (even c) or memory rows (odd c) of k-step c / 2, into slot c % 5
    auto issue = [&](int c) {
      const uint16_t* src = ((c & 1) ? Et : Wt) + (c >> 1) * BK;
      const uint32_t dst = wave_dst + (uint32_t)((c % NSLOT) * SLOT_BYTES);
#pragma unroll
      for (int i = 0; i < G; ++i) dma16(src + off[i], dst + i * 1024);
    };
    floatx16 acc[MF][MT];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int j = 0; j < MT; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    bf16x8 fa[2][MF], fb[2][MT];
    // fragment read n of a sub-step: weight row 0, the memory rows, the other weight rows
    auto read1 = [&](int buf, int sa, int sb, int ss, int n) {
      if (n == 0) fa[buf][0] = *reinterpret_cast<const bf16x8*>(smem + sa + fr_a[ss]);
      else if (n <= MT) fb[buf][n - 1] = *reinterpret_cast<const bf16x8*>(smem + sb + fr_b[ss] + (n - 1) * 32 * BK * 2);
      else fa[buf][n - MT] = *reinterpret_cast<const bf16x8*>(smem + sa + fr_a[ss] + (n - MT) * 32 * BK * 2);
    };
    auto load_frags = [&](int buf, int sa, int sb, int ss) {
#pragma unroll
      for (int n = 0; n < MF + MT; ++n) read1(buf, sa, sb, ss, n);
    };
    auto mfmas = [&](int buf) {
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < MT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
    };
    // one sub-step: the MFMAs of buffer bm, the next sub-step's reads (rs into br) spread
    // evenly, and loads q0 .. q0 + G/2 - 1 of chunk c spread evenly
    auto group = [&](int bm, int br, int rs, int sa, int sb, int c, int q0) {
      constexpr int NM = MF * MT, NR = MF + MT, NL = G / 2;
      const uint16_t* src = ((c & 1) ? Et : Wt) + (c >> 1) * BK;
      const uint32_t dst = wave_dst + (uint32_t)((c % NSLOT) * SLOT_BYTES);
#pragma unroll
      for (int k = 0; k < NM; ++k) {
        if (!(MODE & 4))
          acc[k / MT][k % MT] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[bm][k / MT], fb[bm][k % MT], acc[k / MT][k % MT], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int n = 0; n < NR; ++n)
          if (!(MODE & 2) && (n * NM) / NR == k) read1(br, sa, sb, rs, n);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int l = 0; l < NL; ++l)
          if (!(MODE & 1) && (l * NM) / NL + NM / NL - 1 == k) dma16(src + off[q0 + l], dst + (q0 + l) * 1024);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    for (int c = 0; c < NSLOT; ++c) issue(c);
    wait_vm_lgkm0<3 * G>();  // chunks 0 and 1 (k-step 0) have landed
    lds_barrier();
    load_frags(0, 0, SLOT_BYTES, 0);
    load_frags(1, 0, SLOT_BYTES, 1);
    mfmas(0);
    load_frags(0, 0, SLOT_BYTES, 2);
    mfmas(1);
    load_frags(1, 0, SLOT_BYTES, 3);
    mfmas(0);
    wait_vm_lgkm0<G>();  // chunks 2 and 3 too; chunk 4 may be in flight
    lds_barrier();
    int kt = 1;
    // k-step kt: sub-step 3 of kt - 1 opens it; chunks 2 kt + 3 and 2 kt + 4 go into the
    // slots k-step kt - 1 freed; at its end only chunk 2 kt + 4 may be in flight
    for (; kt + 2 < NK; ++kt) {
      const int sa = ((2 * kt) % NSLOT) * SLOT_BYTES, sb = ((2 * kt + 1) % NSLOT) * SLOT_BYTES;
      __builtin_amdgcn_sched_barrier(0);
      group(1, 0, 0, sa, sb, 2 * kt + 3, 0);
      group(0, 1, 1, sa, sb, 2 * kt + 3, G / 2);
      group(1, 0, 2, sa, sb, 2 * kt + 4, 0);
      group(0, 1, 3, sa, sb, 2 * kt + 4, G / 2);
      __builtin_amdgcn_sched_barrier(0);
      if (MODE & 1) wait_vm_lgkm0<0>();
      else wait_vm_lgkm0<G>();
      lds_barrier();
    }
    for (; kt < NK; ++kt) {  // the last two k-steps: only chunk 2 NK - 1 is left to load
      if (2 * kt + 3 < 2 * NK) issue(2 * kt + 3);
      const int sa = ((2 * kt) % NSLOT) * SLOT_BYTES, sb = ((2 * kt + 1) % NSLOT) * SLOT_BYTES;
      load_frags(0, sa, sb, 0);
      mfmas(1);
      load_frags(1, sa, sb, 1);
      mfmas(0);
      load_frags(0, sa, sb, 2);
      mfmas(1);
      load_frags(1, sa, sb, 3);
      mfmas(0);
      wait_vm_lgkm0<0>();
      lds_barrier();
    }
    mfmas(1);
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int j = 0; j < MT; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) total += acc[i][j][q];
  }
  sink[(int64_t)blockIdx.x * 512 + tid] = total;
  const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (tid == 0) {
    clk[blockIdx.x * 2] = c1 - c0;
    clk[blockIdx.x * 2 + 1] = r1 - r0;
  }
}

template <int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void probe_mainloop_f8_kernel(const uint16_t* __restrict__ W, const uint16_t* __restrict__ E, int rounds,
                              float* __restrict__ sink, uint64_t* __restrict__ clk) {
  constexpr int MF = 4, MT = 4, G = SLOT_BYTES / 1024 / 4;
  __shared__ __attribute__((aligned(16))) char smem[NSLOT * SLOT_BYTES];
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf = wave >> 1, wt = wave & 1;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr)smem;
  const uint32_t wave_dst = lds0 + (uint32_t)(wave * G * 1024);
  const int x = blockIdx.x % 8, w = blockIdx.x / 8;
  const int khalf = lane >> 5;
  const int arow0 = wf * 128 + (lane & 31), brow0 = wt * 128 + (lane & 31);
  // half p of a row: logical chunks 4 p + khalf and 4 p + 2 + khalf
  uint32_t fa_off[2][2], fb_off[2][2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      fa_off[p][h] = (uint32_t)(arow0 * (BK * 2) + (((4 * p + 2 * h + khalf) ^ row_key(arow0)) * 16));
      fb_off[p][h] = (uint32_t)(brow0 * (BK * 2) + (((4 * p + 2 * h + khalf) ^ row_key(brow0)) * 16));
    }
  float total = 0.f;
  for (int r = 0; r < rounds; ++r) {
    const int ttile = ((r / 2) * 8 + x) * 4 + (w & 3), ftile = (r % 2) * 8 + (w >> 2);
    const uint16_t* Wt = W + (int64_t)ftile * 256 * D_MEM;
    const uint16_t* Et = E + (int64_t)ttile * 256 * D_MEM;
    uint32_t off[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int rr = wave * (G * 8) + i * 8 + (lane >> 3);
      off[i] = (uint32_t)rr * D_MEM + (((lane & 7) ^ row_key(rr)) * 8);
    }
    lds_barrier();
    auto issue = [&](int c) {
      const uint16_t* src = ((c & 1) ? Et : Wt) + (c >> 1) * BK;
      const uint32_t dst = wave_dst + (uint32_t)((c % NSLOT) * SLOT_BYTES);
#pragma unroll
      for (int i = 0; i < G; ++i) dma16(src + off[i], dst + i * 1024);
    };
    floatx16 acc[MF][MT];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int j = 0; j < MT; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    v8i fa[2][MF], fb[2][MT];
    auto frag = [&](int base, const uint32_t (&o)[2]) -> v8i {
      const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(smem + base + o[0]);
      const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(smem + base + o[1]);
      return __builtin_shufflevector(__builtin_bit_cast(v4i, lo), __builtin_bit_cast(v4i, hi), 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // fragment n of half p (weight row 0, the memory rows, the other weight rows) into buffer buf
    auto read1 = [&](int buf, int sa, int sb, int p, int n) {
      if (n == 0) fa[buf][0] = frag(sa, fa_off[p]);
      else if (n <= MT) fb[buf][n - 1] = frag(sb + (n - 1) * 32 * BK * 2, fb_off[p]);
      else fa[buf][n - MT] = frag(sa + (n - MT) * 32 * BK * 2, fa_off[p]);
    };
    auto load_frags = [&](int buf, int sa, int sb, int p) {
#pragma unroll
      for (int n = 0; n < MF + MT; ++n) read1(buf, sa, sb, p, n);
    };
    auto mfma = [&](int buf, int i, int j) {
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0, 127, 0,
                                                                 127);
    };
    auto mfmas = [&](int buf) {
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < MT; ++j) mfma(buf, i, j);
    };
    // one half: the 16 MFMAs of buffer bm, the next half's eight fragments (rp into br)
    // one after every second MFMA, and the G loads of chunk c one after every second MFMA
    auto group = [&](int bm, int br, int rp, int sa, int sb, int c) {
      const uint16_t* src = ((c & 1) ? Et : Wt) + (c >> 1) * BK;
      const uint32_t dst = wave_dst + (uint32_t)((c % NSLOT) * SLOT_BYTES);
#pragma unroll
      for (int k = 0; k < MF * MT; ++k) {
        if (!(MODE & 4)) mfma(bm, k / MT, k % MT);
        __builtin_amdgcn_sched_barrier(0);
        if (!(MODE & 2) && (k & 1) == 0) read1(br, sa, sb, rp, k / 2);
        __builtin_amdgcn_sched_barrier(0);
        if (!(MODE & 1) && (k & 1) == 1) dma16(src + off[k / 2], dst + (k / 2) * 1024);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    for (int c = 0; c < NSLOT; ++c) issue(c);
    wait_vm_lgkm0<3 * G>();
    lds_barrier();
    load_frags(0, 0, SLOT_BYTES, 0);
    load_frags(1, 0, SLOT_BYTES, 1);
    mfmas(0);
    wait_vm_lgkm0<G>();
    lds_barrier();
    int kt = 1;
    for (; kt + 2 < NK; ++kt) {
      const int sa = ((2 * kt) % NSLOT) * SLOT_BYTES, sb = ((2 * kt + 1) % NSLOT) * SLOT_BYTES;
      __builtin_amdgcn_sched_barrier(0);
      group(1, 0, 0, sa, sb, 2 * kt + 3);
      group(0, 1, 1, sa, sb, 2 * kt + 4);
      __builtin_amdgcn_sched_barrier(0);
      if (MODE & 1) wait_vm_lgkm0<0>();
      else wait_vm_lgkm0<G>();
      lds_barrier();
    }
    for (; kt < NK; ++kt) {
      if (2 * kt + 3 < 2 * NK) issue(2 * kt + 3);
      const int sa = ((2 * kt) % NSLOT) * SLOT_BYTES, sb = ((2 * kt + 1) % NSLOT) * SLOT_BYTES;
      load_frags(0, sa, sb, 0);
      mfmas(1);
      load_frags(1, sa, sb, 1);
      mfmas(0);
      wait_vm_lgkm0<0>();
      lds_barrier();
    }
    mfmas(1);
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int j = 0; j < MT; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) total += acc[i][j][q];
  }
  sink[(int64_t)blockIdx.x * 512 + tid] = total;
  const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (tid == 0) {
    clk[blockIdx.x * 2] = c1 - c0;
    clk[blockIdx.x * 2 + 1] = r1 - r0;
  }
}

template <int KIND>
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float* __restrict__ sink,
                                                         uint64_t* __restrict__ clk) {
  const int tid = threadIdx.x;
  bf16x8 fa[4], fb[4];
  v8i qa[4], qb[4];  // KIND 1: E4M3 codes (any byte pattern but NaN; 0x7f / 0xff are NaN, cleared)
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t h = (uint32_t)(tid * 8 + e + i * 4096) * 2654435761u;
      fa[i][e] = (__bf16)((float)(h >> 16) / 65536.f - 0.5f);
      fb[i][e] = (__bf16)((float)((h * 2246822519u) >> 16) / 65536.f - 0.5f);
      qa[i][e] = (int)(h & 0xbfbfbfbfu);
      qb[i][e] = (int)((h * 2246822519u) & 0xbfbfbfbfu);
    }
  floatx16 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[j][q] = 0.f;
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (KIND == 0)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[j / 4], fb[j % 4], acc[j], 0, 0, 0);
      else  // E4M3 x E4M3, block scales 127 (2^0)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[j / 4], qb[j % 4], acc[j], 0, 0, 0, 127, 0, 127);
    }
  }
  float total = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) total += acc[j][q];
  __syncthreads();
  const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  sink[(int64_t)blockIdx.x * 256 + tid] = total;
  if (tid == 0) {
    clk[blockIdx.x * 2] = c1 - c0;
    clk[blockIdx.x * 2 + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

// W: device bf16 [4096][1280]; E: device bf16 [engram_probe_mainloop_tokens(rounds)][1280];
// sink: device float [256 * 512]; clk: device uint64 [256 * 2].  256 workgroups (one per CU).
// mode 0..7 (bits: no operand loads, no fragment reads, no MFMAs); waves 4 or 8; rounds even
// and >= 2.  Returns 0, or -1 for bad arguments (nothing launched).
int64_t engram_probe_mainloop_tokens(int32_t rounds) { return (int64_t)((rounds + 1) / 2) * 32 * 256; }

int engram_probe_mainloop(int32_t mode, int32_t waves, const void* W, const void* E, int32_t rounds, float* sink,
                          uint64_t* clk, hipStream_t stream) {
  if (W == nullptr || E == nullptr || sink == nullptr || clk == nullptr || rounds < 2 || rounds % 2 != 0 ||
      mode < 0 || mode > 7 || (waves != 4 && waves != 8))
    return -1;
  const uint16_t* w = (const uint16_t*)W;
  const uint16_t* e = (const uint16_t*)E;
#define ENGRAM_PROBE_CASE(NW_, M_)                                                                   \
  if (waves == NW_ && mode == M_)                                                                    \
    hipLaunchKernelGGL((probe_mainloop_kernel<NW_, M_>), dim3(256), dim3(64 * NW_), 0, stream, w, e, \
                       rounds, sink, clk);
  ENGRAM_PROBE_CASE(4, 0) ENGRAM_PROBE_CASE(4, 1) ENGRAM_PROBE_CASE(4, 2) ENGRAM_PROBE_CASE(4, 3)
  ENGRAM_PROBE_CASE(4, 4) ENGRAM_PROBE_CASE(4, 5) ENGRAM_PROBE_CASE(4, 6) ENGRAM_PROBE_CASE(4, 7)
  ENGRAM_PROBE_CASE(8, 0) ENGRAM_PROBE_CASE(8, 1) ENGRAM_PROBE_CASE(8, 2) ENGRAM_PROBE_CASE(8, 3)
  ENGRAM_PROBE_CASE(8, 4) ENGRAM_PROBE_CASE(8, 5) ENGRAM_PROBE_CASE(8, 6) ENGRAM_PROBE_CASE(8, 7)
#undef ENGRAM_PROBE_CASE
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// The FP8 k-step: the same arguments as engram_probe_mainloop with four waves; mode 0..7.
int engram_probe_mainloop_fp8(int32_t mode, const void* W, const void* E, int32_t rounds, float* sink, uint64_t* clk,
                              hipStream_t stream) {
  if (W == nullptr || E == nullptr || sink == nullptr || clk == nullptr || rounds < 2 || rounds % 2 != 0 ||
      mode < 0 || mode > 7)
    return -1;
  const uint16_t* w = (const uint16_t*)W;
  const uint16_t* e = (const uint16_t*)E;
#define ENGRAM_PROBE_CASE(M_)                                                                               \
  if (mode == M_)                                                                                           \
    hipLaunchKernelGGL((probe_mainloop_f8_kernel<M_>), dim3(256), dim3(256), 0, stream, w, e, rounds, sink, clk);
  ENGRAM_PROBE_CASE(0) ENGRAM_PROBE_CASE(1) ENGRAM_PROBE_CASE(2) ENGRAM_PROBE_CASE(3)
  ENGRAM_PROBE_CASE(4) ENGRAM_PROBE_CASE(5) ENGRAM_PROBE_CASE(6) ENGRAM_PROBE_CASE(7)
#undef ENGRAM_PROBE_CASE
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// kind 0 (bf16) or 1 (FP8); blocks workgroups of 256 threads; sink: device float
// [blocks * 256]; clk: device uint64 [blocks * 2].  Returns 0, or -1 for bad arguments.
int engram_probe_mfma(int32_t kind, int32_t blocks, int32_t iters, float* sink, uint64_t* clk, hipStream_t stream) {
  if (sink == nullptr || clk == nullptr || blocks <= 0 || iters <= 0 || (kind != 0 && kind != 1)) return -1;
  if (kind == 0)
    hipLaunchKernelGGL(probe_mfma_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, stream, iters, sink, clk);
  else
    hipLaunchKernelGGL(probe_mfma_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, iters, sink, clk);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
