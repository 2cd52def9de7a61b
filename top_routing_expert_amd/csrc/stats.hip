// Routing diagnostics of one batch (load-balance report).
//
// Pages: [SyncTax] §5.1 (the per-expert activation frequency and the entropy
// of the routing as the load-balance measure, ideal log2 E bits) and [EP-V4]
// §6.2 (per-expert activation shares against the ideal 1/E).
//   hist[e]       = c_e, the (token, choice) pairs routed to e
//                   (expert_offsets[e+1] - expert_offsets[e], the dispatch's own count)
//   rank_load[r]  = pairs routed to rank r's block of E/R experts
//   stats[0]      = mean over tokens of -sum_e p_e log2 p_e, p = softmax of the
//                   fp32 scores s = z + b over all E experts
//   stats[1]      = mean over tokens of the softmax mass outside the top-presel
//                   experts (order: s desc, e asc); 0 without pre-selection
//   stats[2]      = -sum_e q_e log2 q_e, q = hist / (T k) (zero shares dropped)
//   stats[3]      = E * max_e hist[e] / (T k)  (1 = perfectly even)
//
// gfx950 design: one wave per token (EPL scores per lane), wave-wide max and
// sums by a fixed xor tree; the per-token values go to the workspace and one
// block sums them in a fixed order, so the report is bitwise reproducible.
#include <cmath>

#include "common.h"

namespace moe {

constexpr int kStatsBlock = 1024;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// One wave per token: part[2 t] = entropy (bits), part[2 t + 1] = presel gap.
template <int EPL>
__global__ __launch_bounds__(256) void route_stats_token_kernel(const float* __restrict__ logits,
                                                                const float* __restrict__ bias,
                                                                int T, int E, int presel,
                                                                float* __restrict__ part) {
  extern __shared__ float s_sc[];  // [4 waves][E] scores, for the pre-selection ranks
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + w;
  const bool live = t < T;  // wave-uniform
  float sc[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    sc[i] = -INFINITY;
    if (live && e < E) {
      const float z = logits[(size_t)t * E + e];
      sc[i] = bias ? __fadd_rn(z, bias[e]) : z;
      if (presel) s_sc[w * E + e] = sc[i];
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) m = fmaxf(m, sc[i]);
  m = wave_max(m);
  float ex[EPL], den = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    ex[i] = (live && e < E) ? expf(sc[i] - m) : 0.f;
    den += ex[i];
  }
  den = wave_sum(den);
  float ent = 0.f, kept = 0.f;
  __syncthreads();  // the wave's scores are in LDS
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (!(live && e < E)) continue;
    const float p = ex[i] / den;
    if (p > 0.f) ent -= p * log2f(p);
    if (presel) {
      int rank = 0;  // experts ahead of e in the order (s desc, e asc)
      for (int q = 0; q < E; ++q) {
        const float o = s_sc[w * E + q];
        rank += (o > sc[i]) || (o == sc[i] && q < e);
      }
      if (rank < presel) kept += p;
    }
  }
  ent = wave_sum(ent);
  kept = wave_sum(kept);
  if (live && lane == 0) {
    part[2 * (size_t)t] = ent;
    part[2 * (size_t)t + 1] = presel ? 1.f - kept : 0.f;
  }
}

// Block-wide sum over kStatsBlock threads by a fixed tree.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < kStatsBlock / 64; ++i) r += red[i];
  return r;
}

__global__ __launch_bounds__(kStatsBlock) void route_stats_final_kernel(
    const float* __restrict__ part, int T, int E, int R, int presel,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ roffs,
    int32_t* __restrict__ hist, int32_t* __restrict__ rank_load, float* __restrict__ stats) {
  __shared__ float red[kStatsBlock / 64];
  __shared__ int s_max;
  const int tid = threadIdx.x;
  float se = 0.f, sg = 0.f;
  for (int t = tid; t < T; t += kStatsBlock) {
    se += part[2 * (size_t)t];
    sg += part[2 * (size_t)t + 1];
  }
  se = block_sum(se, red);
  sg = block_sum(sg, red);
  if (tid == 0) s_max = 0;
  const int A = T > 0 ? offs[E] - offs[0] : 0;
  float le = 0.f;
  int mx = 0;
  for (int e = tid; e < E; e += kStatsBlock) {
    const int c = T > 0 ? offs[e + 1] - offs[e] : 0;
    hist[e] = c;
    mx = max(mx, c);
    if (c > 0 && A > 0) {
      const float q = (float)c / (float)A;
      le -= q * log2f(q);
    }
  }
  for (int r = tid; r < R; r += kStatsBlock) rank_load[r] = T > 0 ? roffs[r + 1] - roffs[r] : 0;
  le = block_sum(le, red);  // (its barriers also order s_max's reset before the atomics)
  atomicMax(&s_max, mx);
  __syncthreads();
  if (tid == 0) {
    stats[0] = T > 0 ? se / (float)T : 0.f;
    stats[1] = (T > 0 && presel) ? sg / (float)T : 0.f;
    stats[2] = le;
    stats[3] = A > 0 ? (float)E * (float)s_max / (float)A : 0.f;
  }
}

size_t route_stats_ws_bytes(const moe_config& c) { return (size_t)c.T * 2 * sizeof(float); }

hipError_t launch_route_stats(const moe_config& c, const float* logits, const float* bias,
                              const int32_t* offs, const int32_t* roffs, int32_t* hist,
                              int32_t* rank_load, float* stats, void* ws, hipStream_t st) {
  float* part = static_cast<float*>(ws);
  if (c.T > 0) {
    const dim3 grid(div_up(c.T, 4));
    const size_t lds = c.presel ? 4 * (size_t)c.E * sizeof(float) : 0;
    if (c.E <= 64)
      route_stats_token_kernel<1><<<grid, 256, lds, st>>>(logits, bias, c.T, c.E, c.presel, part);
    else if (c.E <= 256)
      route_stats_token_kernel<4><<<grid, 256, lds, st>>>(logits, bias, c.T, c.E, c.presel, part);
    else
      route_stats_token_kernel<16><<<grid, 256, lds, st>>>(logits, bias, c.T, c.E, c.presel, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  route_stats_final_kernel<<<1, kStatsBlock, 0, st>>>(part, c.T, c.E, c.ep_ranks, c.presel, offs,
                                                      roffs, hist, rank_load, stats);
  return hipGetLastError();
}

}  // namespace moe
