// Weighted combine back to token order:
//   out[t] = sum_{j=0..k-1} topk_w[t, j] * y_perm[slot_of[t*k + j]]   (fp32, j ascending)
//
// Pages: [SyncTax] §2.3 (each token's k expert outputs are summed with their
// gate weights on the token's home device).
//
// gfx950 design: one wave per token, 16-byte vector gathers of the k expert
// rows (each row contiguous; 8-16 gathers per lane in flight), fp32 FMAs
// in a fixed j order, one 16-byte store per lane and vector.  HBM traffic is the algorithmic minimum: every y_perm row is read
// once and every out row written once.
#include "common.h"

namespace moe {

constexpr int kMaxKC = 16;

// KC: k rounded up to 1, 2, 4, 8 or kMaxKC; U: 16-byte vectors per lane in
// flight per expert row, so that every lane keeps 8 (16 for k = 8) loads in
// flight and a token's row is read in few memory round trips.  The y_perm
// rows are read exactly once, with non-temporal loads (measured after the down
// GEMM: T8192-d7168-k8 235 -> 212 us, and 192 us with U = 2 for k = 8;
// T16384-d5120-k2 89 -> 81 us; non-temporal stores of out were slower).
// wave >= 0: only the tokens whose highest-numbered chosen expert lies in
// experts [wave * per, (wave + 1) * per) -- the tokens whose last expert wave
// that is (the waved layer combines each token once, after that wave).
template <int KC, int U>
__global__ __launch_bounds__(256) void combine_bf16_kernel(const u32x4* __restrict__ y,
                                                           const int32_t* __restrict__ slot_of,
                                                           const float* __restrict__ topk_w,
                                                           u32x4* __restrict__ out, int T, int k,
                                                           int row_vecs,
                                                           const int32_t* __restrict__ topk_idx,
                                                           int wave, int per) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  if (wave >= 0) {  // wave-uniform test of the token's last expert wave
    int e = lane < k ? topk_idx[(size_t)t * k + lane] : 0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) e = max(e, __shfl_xor(e, o));
    if (e / per != wave) return;
  }
  int p = 0;
  float g = 0.f;
  if (lane < k) {
    p = slot_of[(size_t)t * k + lane];
    p = p < 0 ? 0 : (p >= T * k ? T * k - 1 : p);  // keep every access in bounds
    g = topk_w[(size_t)t * k + lane];
  }
  int pj[KC];
  float gj[KC];
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    pj[j] = __shfl(p, j);
    gj[j] = __shfl(g, j);
  }
  for (int v0 = lane; v0 < row_vecs; v0 += 64 * U) {
    u32x4 w[U][KC];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < KC; ++j)
        if (j < k && v0 + 64 * u < row_vecs)  // read once: a streaming (non-temporal) load
          w[u][j] = __builtin_nontemporal_load(&y[(size_t)pj[j] * row_vecs + v0 + 64 * u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (v0 + 64 * u >= row_vecs) break;
      float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        if (j < k) {
          a[0] = fmaf(gj[j], bf16_lo(w[u][j].x), a[0]);
          a[1] = fmaf(gj[j], bf16_hi(w[u][j].x), a[1]);
          a[2] = fmaf(gj[j], bf16_lo(w[u][j].y), a[2]);
          a[3] = fmaf(gj[j], bf16_hi(w[u][j].y), a[3]);
          a[4] = fmaf(gj[j], bf16_lo(w[u][j].z), a[4]);
          a[5] = fmaf(gj[j], bf16_hi(w[u][j].z), a[5]);
          a[6] = fmaf(gj[j], bf16_lo(w[u][j].w), a[6]);
          a[7] = fmaf(gj[j], bf16_hi(w[u][j].w), a[7]);
        }
      }
      u32x4 o;
      o.x = pack_bf16x2(a[0], a[1]);
      o.y = pack_bf16x2(a[2], a[3]);
      o.z = pack_bf16x2(a[4], a[5]);
      o.w = pack_bf16x2(a[6], a[7]);
      out[(size_t)t * row_vecs + v0 + 64 * u] = o;
    }
  }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(const float4* __restrict__ y,
                                                          const int32_t* __restrict__ slot_of,
                                                          const float* __restrict__ topk_w,
                                                          float4* __restrict__ out, int T, int k,
                                                          int row_vecs) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int p = 0;
  float g = 0.f;
  if (lane < k) {
    p = slot_of[(size_t)t * k + lane];
    p = p < 0 ? 0 : (p >= T * k ? T * k - 1 : p);  // keep every access in bounds
    g = topk_w[(size_t)t * k + lane];
  }
  int pj[kMaxKC];
  float gj[kMaxKC];
#pragma unroll
  for (int j = 0; j < kMaxKC; ++j) {
    pj[j] = __shfl(p, j);
    gj[j] = __shfl(g, j);
  }
  for (int v = lane; v < row_vecs; v += 64) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < kMaxKC; ++j) {
      if (j < k) {
        const float4 w = y[(size_t)pj[j] * row_vecs + v];
        a.x = fmaf(gj[j], w.x, a.x);
        a.y = fmaf(gj[j], w.y, a.y);
        a.z = fmaf(gj[j], w.z, a.z);
        a.w = fmaf(gj[j], w.w, a.w);
      }
    }
    out[(size_t)t * row_vecs + v] = a;
  }
}

hipError_t launch_combine(const moe_config& c, const void* y_perm, const int32_t* slot_of,
                          const float* topk_w, void* out, hipStream_t st,
                          const int32_t* topk_idx, int wave, int per) {
  const dim3 grid(div_up(c.T, 4));
  if (c.dtype == MOE_BF16) {
    auto* yv = static_cast<const u32x4*>(y_perm);
    auto* ov = static_cast<u32x4*>(out);
    const int rv = c.d / 8;
#define MOE_COMBINE(KC, U)                                                               \
  combine_bf16_kernel<KC, U><<<grid, 256, 0, st>>>(yv, slot_of, topk_w, ov, c.T, c.k, rv, \
                                                   topk_idx, wave, per)
    if (c.k <= 1)
      MOE_COMBINE(1, 8);
    else if (c.k <= 2)
      MOE_COMBINE(2, 4);
    else if (c.k <= 4)
      MOE_COMBINE(4, 2);
    else if (c.k <= 8)
      MOE_COMBINE(8, 2);
    else
      MOE_COMBINE(kMaxKC, 1);
#undef MOE_COMBINE
  } else {
    combine_f32_kernel<<<grid, 256, 0, st>>>(static_cast<const float4*>(y_perm), slot_of, topk_w,
                                             static_cast<float4*>(out), c.T, c.k, c.d / 4);
  }
  return hipGetLastError();
}

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  fill_i32_kernel<<<div_up(n, 256), 256, 0, st>>>(p, n, v);
  return hipGetLastError();
}

}  // namespace moe
