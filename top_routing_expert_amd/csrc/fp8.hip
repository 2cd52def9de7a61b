// Per-token FP8 compression of the dispatch payload.
//
// Pages: [SyncTax] §3.1 -- the expert inputs / outputs that cross the
// all-to-all are quantised to FP8 per token: every token's vector gets its
// own min / max and an affine map, so one outlier does not widen the range of
// every token, and the payload shrinks to one byte per element.
//
// quantize: one row per RT threads (RT = 256 for rows of more than 1024
//   elements, else one wave), each thread up to 4 vectors of 8 bf16 that stay
//   in registers: the row's min / max (wave tree, then LDS across the row's
//   waves), then centre z = (max + min) / 2 and scale s = ((max - min) / 2) /
//   448 in float32, v = (x - z) / s (0 for a constant row), clamped to +-448
//   and rounded to E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa
//   bits), nearest with ties to the even code.  Spreading a row over a whole
//   block keeps several waves per SIMD busy on the per-element divide and
//   encode even when there are only a few rows per CU.
// dequantize: one expert-ordered row p per RT threads: the codes of token
//   src_of[p] / k come back as bf16(code * s + z) (float32 multiply, float32
//   add, bf16 round to nearest even) -- the receiver's x_perm.  Every thread
//   issues all of its code loads before it decodes.
// Every step is an exactly specified float32 operation, so the codes, scales
// and decoded rows are bit-exact against a float32 replay.  The default
// contraction would fuse a multiply and the add after it into one fma (one
// rounding instead of two): contraction is off in this file, and its float
// operations are written here, not taken from header helpers compiled with
// contraction on.
#include <cmath>

#include "common.h"
#include "fp8_codec.h"

#pragma clang fp contract(off)

namespace moe {

__device__ __forceinline__ float f32_add(float a, float b) { return a + b; }
__device__ __forceinline__ float f32_sub(float a, float b) { return a - b; }
__device__ __forceinline__ float f32_mul(float a, float b) { return a * b; }
__device__ __forceinline__ float f32_div(float a, float b) { return a / b; }  // correctly rounded

constexpr int kF8VecsPerThread = 4;  // d <= 256 threads * 4 vectors * 8 = 8192
__device__ __forceinline__ float f8_wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float f8_wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// RT threads per row (64 or 256), 256 / RT rows per block.
template <int RT>
__global__ __launch_bounds__(256) void fp8_quantize_rows_kernel(const u32x4* __restrict__ x, int T,
                                                                int nvec,
                                                                u32x2* __restrict__ codes,
                                                                float* __restrict__ scale_zero) {
  constexpr int RB = 256 / RT, WPR = RT / 64;
  __shared__ float s_lo[4], s_hi[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i0 = tid % RT;
  const int t = blockIdx.x * RB + tid / RT;
  const bool live = t < T;  // uniform over the row's threads
  const u32x4* row = x + (size_t)(live ? t : 0) * nvec;
  u32x4 r[kF8VecsPerThread];
#pragma unroll
  for (int i = 0; i < kF8VecsPerThread; ++i) {
    const int v = i0 + RT * i;
    if (live && v < nvec) r[i] = row[v];
  }
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int i = 0; i < kF8VecsPerThread; ++i) {
    const int v = i0 + RT * i;
    if (live && v < nvec) {
      const uint32_t wd[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float a = bf16_lo(wd[q]), b = bf16_hi(wd[q]);
        lo = fminf(lo, fminf(a, b));
        hi = fmaxf(hi, fmaxf(a, b));
      }
    }
  }
  lo = f8_wave_min(lo);
  hi = f8_wave_max(hi);
  if constexpr (WPR > 1) {  // RB == 1: the block is one row
    if (lane == 0) {
      s_lo[w] = lo;
      s_hi[w] = hi;
    }
    __syncthreads();
    lo = s_lo[0];
    hi = s_hi[0];
#pragma unroll
    for (int q = 1; q < WPR; ++q) {
      lo = fminf(lo, s_lo[q]);
      hi = fmaxf(hi, s_hi[q]);
    }
  }
  if (!live) return;
  const float z = f32_mul(f32_add(hi, lo), 0.5f);
  const float s = f32_div(f32_mul(f32_sub(hi, lo), 0.5f), kF8Max);
  if (i0 == 0) {
    scale_zero[2 * (size_t)t] = s;
    scale_zero[2 * (size_t)t + 1] = z;
  }
  u32x2* out = codes + (size_t)t * nvec;
#pragma unroll
  for (int i = 0; i < kF8VecsPerThread; ++i) {
    const int v = i0 + RT * i;
    if (v < nvec) {
      const uint32_t wd[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
      uint32_t c[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float xv = (q & 1) ? bf16_hi(wd[q >> 1]) : bf16_lo(wd[q >> 1]);
        float y = s > 0.f ? f32_div(f32_sub(xv, z), s) : 0.f;
        y = fminf(fmaxf(y, -kF8Max), kF8Max);
        c[q] = e4m3_encode(y);
      }
      u32x2 pk;
      pk.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
      pk.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
      out[v] = pk;
    }
  }
}

template <int RT>
__global__ __launch_bounds__(256) void fp8_dequantize_gather_kernel(
    const u32x2* __restrict__ codes, const int32_t* __restrict__ src_of,
    const float* __restrict__ scale_zero, int rows, int k, int T, int nvec,
    u32x4* __restrict__ x_perm) {
  constexpr int RB = 256 / RT;
  const int tid = threadIdx.x, i0 = tid % RT;
  const int p = blockIdx.x * RB + tid / RT;
  if (p >= rows) return;
  const int t = min(max(src_of[p] / k, 0), T - 1);  // a malformed index stays in bounds
  const float s = scale_zero[2 * (size_t)t], z = scale_zero[2 * (size_t)t + 1];
  const u32x2* row = codes + (size_t)t * nvec;
  u32x4* out = x_perm + (size_t)p * nvec;
  u32x2 c[kF8VecsPerThread];
#pragma unroll
  for (int i = 0; i < kF8VecsPerThread; ++i) {
    const int v = i0 + RT * i;
    if (v < nvec) c[i] = row[v];
  }
#pragma unroll
  for (int i = 0; i < kF8VecsPerThread; ++i) {
    const int v = i0 + RT * i;
    if (v < nvec) {
      float f[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t b = ((q < 4 ? c[i].x : c[i].y) >> (8 * (q & 3))) & 0xFFu;
        f[q] = f32_add(f32_mul(e4m3_decode(b), s), z);
      }
      u32x4 o;
      o.x = pack_bf16x2(f[0], f[1]);
      o.y = pack_bf16x2(f[2], f[3]);
      o.z = pack_bf16x2(f[4], f[5]);
      o.w = pack_bf16x2(f[6], f[7]);
      out[v] = o;
    }
  }
}

bool fp8_row_supported(const moe_config& c) {
  return c.dtype == MOE_BF16 && c.d % 8 == 0 && c.d / 8 <= 256 * kF8VecsPerThread;
}

// Rows of more than 1024 elements get a whole block, shorter ones one wave.
static bool fp8_wide_rows(int nvec) { return nvec > 64 * kF8VecsPerThread / 2; }

hipError_t launch_fp8_quantize(const moe_config& c, const void* x, void* codes, float* scale_zero,
                               hipStream_t st) {
  const int nvec = c.d / 8;
  const auto* xs = static_cast<const u32x4*>(x);
  auto* cs = static_cast<u32x2*>(codes);
  if (fp8_wide_rows(nvec))
    fp8_quantize_rows_kernel<256><<<c.T, 256, 0, st>>>(xs, c.T, nvec, cs, scale_zero);
  else
    fp8_quantize_rows_kernel<64><<<div_up(c.T, 4), 256, 0, st>>>(xs, c.T, nvec, cs, scale_zero);
  return hipGetLastError();
}

hipError_t launch_fp8_dequantize(const moe_config& c, const void* codes, const int32_t* src_of,
                                 const float* scale_zero, void* x_perm, hipStream_t st) {
  const int rows = c.T * c.k, nvec = c.d / 8;
  const auto* cs = static_cast<const u32x2*>(codes);
  auto* out = static_cast<u32x4*>(x_perm);
  if (fp8_wide_rows(nvec))
    fp8_dequantize_gather_kernel<256><<<rows, 256, 0, st>>>(cs, src_of, scale_zero, rows, c.k, c.T,
                                                           nvec, out);
  else
    fp8_dequantize_gather_kernel<64><<<div_up(rows, 4), 256, 0, st>>>(cs, src_of, scale_zero, rows,
                                                                     c.k, c.T, nvec, out);
  return hipGetLastError();
}

}  // namespace moe
