// quant.hip -- per-row FP8 (OCP E4M3) quantization.
// "Conditional Memory via Scalable Lookup", section 2.4: the projections may run as one
// FP8 matrix multiplication.  The pages name no format or scaling; this library uses
// E4M3 (the format gfx950's FP8 matrix instructions read) with one fp32 scale per row
// of each operand:
//   s[r]      = max_c |x[r][c]| / 448          (1 for an all-zero row)
//   code[r][c] = E4M3 value nearest to x[r][c] / s[r], ties to the even code,
//                magnitudes at or above 448 saturated to 448
// so that the largest element of every row lands on the largest finite code.
//
// E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 holds the
// subnormals m * 2^-9; 0x7E = 1.75 * 2^8 = 448 is the largest finite value.  This is
// the format of gfx950's FP8 conversion and matrix instructions.
//
// One wavefront per row.  Rows of up to 4096 columns are read once into registers
// (R 8-value chunks per lane) and encoded from there; longer rows are read twice (max,
// then codes), the second read mostly from cache.  Optionally the row's gains are
// folded in first (x[r][c] = (grow[r] * x[r][c]) * gcol[c] in fp32) and the sum of
// squares of the dequantized row is returned (the memory vector's RMS for the gate).
#include "engram_internal.h"

namespace engram {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_at(const uint16_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

template <bool BF16>
__device__ __forceinline__ void load8(const void* row, int c8, float* x) {
  if constexpr (BF16) {
    const u32x4 v = *reinterpret_cast<const u32x4*>((const uint16_t*)row + c8 * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(v[i] << 16);
      x[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  } else {
    const u32x4 a = *reinterpret_cast<const u32x4*>((const float*)row + c8 * 8);
    const u32x4 b = *reinterpret_cast<const u32x4*>((const float*)row + c8 * 8 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = __uint_as_float(a[i]);
      x[4 + i] = __uint_as_float(b[i]);
    }
  }
}

// rows x cols (cols % 16 == 0), a wavefront per row; grow/gcol optional gains.
template <bool BF16>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* src, int64_t rows, int32_t cols,
                                                         const void* grow, const void* gcol, uint8_t* codes,
                                                         float* scales, float* sumsq) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;  // uniform per wavefront
  const int lane = threadIdx.x & 63;
  const int n8 = cols / 8;
  const char* row = (const char*)src + r * (int64_t)cols * (BF16 ? 2 : 4);
  auto gain_r = [&]() -> float {
    if (grow == nullptr) return 1.f;
    return BF16 ? bf16_at((const uint16_t*)grow, r) : ((const float*)grow)[r];
  };
  const float gr = gain_r();
  auto fold = [&](int c8, float* x) {
    load8<BF16>(row, c8, x);
    if (grow != nullptr || gcol != nullptr) {
      float gc[8];
      if (gcol != nullptr) load8<BF16>(gcol, c8, gc);
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = (gr * x[i]) * (gcol != nullptr ? gc[i] : 1.f);
    }
  };
  float mx = 0.f;
  for (int c8 = lane; c8 < n8; c8 += 64) {
    float x[8];
    fold(c8, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(x[i]));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  const float s = mx > 0.f ? mx / 448.0f : 1.0f;
  float ss = 0.f;
  uint8_t* out = codes + r * (int64_t)cols;
  for (int c16 = lane; c16 < cols / 16; c16 += 64) {
    u32x4 o;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float x[8];
      fold(2 * c16 + h, x);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint32_t w = e4m3_pack4(x[4 * q] / s, x[4 * q + 1] / s, x[4 * q + 2] / s, x[4 * q + 3] / s);
        ss += sumsq4(w, s);
        o[2 * h + q] = w;
      }
    }
    *reinterpret_cast<u32x4*>(out + c16 * 16) = o;
  }
  if (sumsq != nullptr) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  }
  if (lane == 0) {
    scales[r] = s;
    if (sumsq != nullptr) sumsq[r] = ss;
  }
}

// Rows held in registers: lane l owns 8-value chunks l, l + 64, .., l + 64 (R - 1).
template <bool BF16, int R>
__global__ __launch_bounds__(256) void quant_rows_reg_kernel(const void* src, int64_t rows, int32_t cols,
                                                             const void* grow, const void* gcol, uint8_t* codes,
                                                             float* scales, float* sumsq) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;  // uniform per wavefront
  const int lane = threadIdx.x & 63;
  const int n8 = cols / 8;
  const char* row = (const char*)src + r * (int64_t)cols * (BF16 ? 2 : 4);
  const float gr = grow == nullptr ? 1.f
                                   : (BF16 ? bf16_at((const uint16_t*)grow, r) : ((const float*)grow)[r]);
  float x[R][8];
  float mx = 0.f;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int c8 = lane + 64 * k;
    if (c8 < n8) {
      load8<BF16>(row, c8, x[k]);
      if (grow != nullptr || gcol != nullptr) {
        float gc[8];
        if (gcol != nullptr) load8<BF16>(gcol, c8, gc);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[k][i] = (gr * x[k][i]) * (gcol != nullptr ? gc[i] : 1.f);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(x[k][i]));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  const float s = mx > 0.f ? mx / 448.0f : 1.0f;
  float ss = 0.f;
  uint8_t* out = codes + r * (int64_t)cols;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int c8 = lane + 64 * k;
    if (c8 < n8) {
      uint32_t w[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float* v = x[k] + 4 * q;
        w[q] = e4m3_pack4(v[0] / s, v[1] / s, v[2] / s, v[3] / s);
        ss += sumsq4(w[q], s);
      }
      *reinterpret_cast<uint2*>(out + c8 * 8) = make_uint2(w[0], w[1]);
    }
  }
  if (sumsq != nullptr) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  }
  if (lane == 0) {
    scales[r] = s;
    if (sumsq != nullptr) sumsq[r] = ss;
  }
}

template <bool BF16>
void launch_rows(const void* src, int64_t rows, int32_t cols, const void* grow, const void* gcol, uint8_t* codes,
                 float* scales, float* sumsq, hipStream_t s) {
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  const int per_lane = (cols / 8 + 63) / 64;
  if (per_lane <= 1)
    hipLaunchKernelGGL((quant_rows_reg_kernel<BF16, 1>), grid, block, 0, s, src, rows, cols, grow, gcol, codes,
                       scales, sumsq);
  else if (per_lane <= 2)
    hipLaunchKernelGGL((quant_rows_reg_kernel<BF16, 2>), grid, block, 0, s, src, rows, cols, grow, gcol, codes,
                       scales, sumsq);
  else if (per_lane <= 3)
    hipLaunchKernelGGL((quant_rows_reg_kernel<BF16, 3>), grid, block, 0, s, src, rows, cols, grow, gcol, codes,
                       scales, sumsq);
  else if (per_lane <= 4)
    hipLaunchKernelGGL((quant_rows_reg_kernel<BF16, 4>), grid, block, 0, s, src, rows, cols, grow, gcol, codes,
                       scales, sumsq);
  else if (per_lane <= 8)
    hipLaunchKernelGGL((quant_rows_reg_kernel<BF16, 8>), grid, block, 0, s, src, rows, cols, grow, gcol, codes,
                       scales, sumsq);
  else
    hipLaunchKernelGGL(quant_rows_kernel<BF16>, grid, block, 0, s, src, rows, cols, grow, gcol, codes, scales,
                       sumsq);
}

}  // namespace

void launch_quant_rows(const void* src, bool bf16, int64_t rows, int32_t cols, const void* grow, const void* gcol,
                       uint8_t* codes, float* scales, float* sumsq, hipStream_t s) {
  if (bf16) launch_rows<true>(src, rows, cols, grow, gcol, codes, scales, sumsq, s);
  else launch_rows<false>(src, rows, cols, grow, gcol, codes, scales, sumsq, s);
}

}  // namespace engram
