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
// subnormals m * 2^-9; 0x7E = 1.75 * 2^8 = 448 is the largest finite value.
//
// One wavefront per row.  Rows are read twice (max, then codes) as 16-byte chunks; the
// second read hits L2 for the row just scanned.  Optionally the row's gains are folded
// in first (x[r][c] = (grow[r] * x[r][c]) * gcol[c] in fp32) and the sum of squares of
// the dequantized row is returned (the memory vector's RMS for the gate).
#include "engram_internal.h"

namespace engram {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// E4M3 code of v (round to nearest even, saturating), from v's binary32 fields.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t mag = u & 0x7fffffffu;
  if (mag >= 0x43e00000u) return sign | 0x7eu;  // |v| >= 448
  const int ex = (int)(mag >> 23) - 127;         // |v| in [2^ex, 2^(ex+1)) (fp32 normals)
  if (ex < -6) {
    // subnormal range of E4M3: spacing 2^-9; 8 * 2^-9 is the smallest normal (code 0x08)
    const float r = __builtin_rintf(__builtin_ldexpf(__uint_as_float(mag), 9));
    return sign | (uint32_t)r;
  }
  // normal range: 8 steps of 2^(ex-3) per binade; r in [8, 16]
  uint32_t r = (uint32_t)__builtin_rintf(__builtin_ldexpf(__uint_as_float(mag), 3 - ex));
  int e = ex;
  if (r == 16u) {
    r = 8u;
    ++e;
  }
  const uint32_t code = ((uint32_t)(e + 7) << 3) | (r - 8u);
  return sign | (code > 0x7eu ? 0x7eu : code);
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float v = e == 0 ? __builtin_ldexpf((float)m, -9) : __builtin_ldexpf((float)(8u + m), (int)e - 10);
  return (c & 0x80u) ? -v : v;
}

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
        uint32_t w = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t c = e4m3_code(x[4 * q + b] / s);
          const float d = e4m3_value(c) * s;
          ss += d * d;
          w |= c << (8 * b);
        }
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

}  // namespace

void launch_quant_rows(const void* src, bool bf16, int64_t rows, int32_t cols, const void* grow, const void* gcol,
                       uint8_t* codes, float* scales, float* sumsq, hipStream_t s) {
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (bf16)
    hipLaunchKernelGGL(quant_rows_kernel<true>, grid, dim3(256), 0, s, src, rows, cols, grow, gcol, codes, scales,
                       sumsq);
  else
    hipLaunchKernelGGL(quant_rows_kernel<false>, grid, dim3(256), 0, s, src, rows, cols, grow, gcol, codes, scales,
                       sumsq);
}

}  // namespace engram
