// Router: gate GEMM z = x . Wr^T, then scores, (group-limited) top-k and gates.
//
// Pages: [EP-V4] §2.1 (each token's logits over all experts, then local top-2
// and softmax gates), §3.2 (max subtraction before the exponential; partial
// sort to the top-8 and an exact softmax over those); [V4-overlap] EP-on-IB
// section (experts chosen only within the best groups/nodes).
//
// gfx950 design
//  * Gate GEMM (bf16), E <= 16: a stream over x, see router_skinny_bf16_kernel.
//  * Gate GEMM (bf16), E > 16: MFMA 16x16x32, experts on the M side (A operand, staged
//    through LDS per 64-wide K chunk), tokens on the N side (B operand, read
//    straight from HBM into registers: every x row is used by exactly one
//    wave, so it never needs LDS).  A block is 4 waves x 16 tokens and up to
//    256 experts.  Short batches are split along d into `splits` partial
//    products that the top-k kernel sums in a fixed order, so logits stay
//    bitwise reproducible (no float atomics) while the grid still covers the
//    256 CUs.
//  * Top-k: a group of LPT = min(64, pow2 >= E) lanes per token (32 for
//    64 < E <= 256 with at most 32 groups); each lane holds E/LPT scores.
//    Every selection round is one argmax over 64-bit keys (order-preserving
//    score bits, then inverted index), reduced with xor shuffles: highest
//    score wins, ties go to the lowest expert index.
#include "common.h"

namespace moe {

constexpr int kMaxSplits = 16;  // split-K partials of the router GEMM (summed by top-k)

typedef int i32x4 __attribute__((ext_vector_type(4)));

// ============================================================== gate GEMM bf16
// One K chunk = 64 bf16 of every row.  Inside a chunk lane group g = lane/16
// owns k in [16g, 16g+16) (two 16-byte pieces); the two MFMA k-slabs take the
// first and second piece.  A and B use the same assignment, so the products
// pair up correctly whatever the hardware's k order inside one MFMA is.
template <int EC>
__global__ __launch_bounds__(256) void router_gemm_bf16_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ wr,
                                                               float* __restrict__ dst, int T, int d,
                                                               int E, int splits) {
  constexpr int NF = EC / 16;                         // expert fragments per wave
  constexpr int WLOADS = (EC * 8 + 255) / 256;        // 16-byte pieces per thread per chunk
  __shared__ u32x4 sW[2][EC * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e0 = blockIdx.z * EC;
  const int nch = d >> 6;
  const int c_beg = (int)((long)blockIdx.y * nch / splits);
  const int c_end = (int)((long)(blockIdx.y + 1) * nch / splits);
  const int g = lane >> 4;

  const int tok = blockIdx.x * 64 + wave * 16 + (lane & 15);
  const u32x4* xrow = reinterpret_cast<const u32x4*>(x + (size_t)min(tok, T - 1) * d);

  // W chunk loader: piece i of this thread covers row (p >> 3), piece (p & 7).
  const u32x4* wrow[WLOADS];
  int wdst[WLOADS];
  bool wact[WLOADS];
#pragma unroll
  for (int i = 0; i < WLOADS; ++i) {
    const int p = tid + i * 256;
    wact[i] = p < EC * 8;
    const int r = p >> 3, q = p & 7;
    const int er = min(e0 + r, E - 1);
    wrow[i] = reinterpret_cast<const u32x4*>(wr + (size_t)er * d) + q;
    wdst[i] = r * 8 + (q ^ (r & 7));
  }

  f32x4 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Chunks are loaded two ahead through a ring of three register slots:
  // chunk c sits in slot (c - c_beg) % 3, its W half in LDS stage (c - c_beg) & 1.
  // In iteration c, slot (c+2) is refilled (its chunk c-1 is consumed), chunk
  // c is computed, then chunk c+1's W moves to the other LDS stage.  The loop
  // is unrolled by three so that every slot index is static.
  u32x4 wreg[3][WLOADS];
  u32x4 xr[3][2];
  auto issue = [&](int slot, int c) {
#pragma unroll
    for (int i = 0; i < WLOADS; ++i)
      if (wact[i]) wreg[slot][i] = wrow[i][c * 8];
    xr[slot][0] = xrow[c * 8 + 2 * g];
    xr[slot][1] = xrow[c * 8 + 2 * g + 1];
  };
  if (c_beg < c_end) {
    issue(0, c_beg);
    if (c_beg + 1 < c_end) issue(1, c_beg + 1);
#pragma unroll
    for (int i = 0; i < WLOADS; ++i)
      if (wact[i]) sW[0][wdst[i]] = wreg[0][i];
  }
  __syncthreads();

  for (int c0 = c_beg; c0 < c_end; c0 += 3) {
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const int c = c0 + r;
      if (c < c_end) {  // block-uniform
        const int st = (c - c_beg) & 1;
        if (c + 2 < c_end) issue((r + 2) % 3, c + 2);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 b = as_bf16x8(xr[r][s]);
          const int q = 2 * g + s;
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            const int row = f * 16 + (lane & 15);
            const bf16x8 a = as_bf16x8(sW[st][row * 8 + (q ^ (row & 7))]);
            acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[f], 0, 0, 0);
          }
        }
        if (c + 1 < c_end) {
#pragma unroll
          for (int i = 0; i < WLOADS; ++i)
            if (wact[i]) sW[st ^ 1][wdst[i]] = wreg[(r + 1) % 3][i];
        }
        __syncthreads();
      }
    }
  }

  // acc[f][i] = z[token = lane&15][expert = e0 + 16f + 4(lane>>4) + i]
  if (tok < T) {
    float* drow = dst + ((size_t)blockIdx.y * T + tok) * E;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = e0 + f * 16 + 4 * g + i;
        if (e < E) drow[e] = acc[f][i];
      }
    }
  }
}

// ======================================================= gate GEMM bf16, E <= 16
// Few experts: the GEMM is a stream over x with E flop per byte.  MFMA
// 16x16x32 with the experts on the A side (rows past E repeat the last expert
// and are not stored) and the 16 tokens of a wave on the B side.
//  * x is read in whole 128-byte lines: one load covers 8 token rows x 128 B
//    (64 k), two loads a wave's 16 rows.  (The B-operand layout itself would
//    read 64 B of 16 rows per load; those half-line steps measured 30 % slower
//    on the T16384-d5120 router.)  Each wave writes its two loads to a
//    private 2 KB LDS tile (16-byte pieces swizzled by (row >> 1) & 7, so
//    neither the row-wise writes nor the column-wise fragment reads conflict)
//    and reads back the B fragments of the two MFMAs of the 64 k.
//  * The A fragments (Wr, a few hundred KB, L1/L2-resident) are loaded in
//    MFMA layout.  Lane group g = lane/16 takes piece 4h + g of the 64 k for
//    MFMA h on both operands, so the products pair up whatever the hardware's
//    k order inside one MFMA is.
//  * Loads run kSkinnyDepth k-pairs ahead; no barriers (a wave reads only its
//    own LDS tile).
constexpr int kSkinnyDepth = 6;

// Raw buffer resource over `bytes` bytes (word 3: raw, untyped, gfx950).
__device__ __forceinline__ i32x4 router_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

// 16 bytes per lane; issued and waited for explicitly (see below).
__device__ __forceinline__ u32x4 rload_async(i32x4 rsrc, uint32_t voff, int soff) {
  u32x4 v;
  asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen" : "=v"(v) : "v"(voff), "s"(rsrc), "s"(soff));
  return v;
}
// The same with the non-temporal hint, for the x stream: those lines are not
// allocated in the MALL, so the dirty lines the previous kernels left there
// are not written back while the router streams (T16384-d5120 after 1 GiB of
// writes: 72 -> 40 us; in the layer step 59 -> 46 us).
__device__ __forceinline__ u32x4 rload_async_nt(i32x4 rsrc, uint32_t voff, int soff) {
  u32x4 v;
  asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen nt" : "=v"(v) : "v"(voff), "s"(rsrc), "s"(soff));
  return v;
}
template <int N>
__device__ __forceinline__ void rwait4(u32x4& a, u32x4& b, u32x4& c, u32x4& d) {
  asm volatile("s_waitcnt vmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "n"(N));
}

__global__ __launch_bounds__(256) void router_skinny_bf16_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ wr,
                                                                 float* __restrict__ dst, int T,
                                                                 int d, int E, int splits) {
  constexpr int P = kSkinnyDepth;
  __shared__ u32x4 tile[4][128];  // per wave: 16 rows x 8 pieces
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tok0 = (blockIdx.x * 4 + wave) * 16;
  const int nkp = d >> 6;  // k-pairs of 64
  const int kb = (int)((long)blockIdx.y * nkp / splits);
  const int ke = (int)((long)(blockIdx.y + 1) * nkp / splits);
  // T * d and E * d are < 2^31 elements (checked by the C ABI): byte offsets fit 32 bits
  const i32x4 xs = router_rsrc(x, (uint32_t)T * (uint32_t)d * 2u);
  const i32x4 ws = router_rsrc(wr, (uint32_t)E * (uint32_t)d * 2u);
  const int lr = lane >> 3, lp = lane & 7;  // x load: row lr (+8), piece lp of the 128 B
  const uint32_t xo0 = ((uint32_t)min(tok0 + lr, T - 1) * (uint32_t)d + 8u * lp) * 2u;
  const uint32_t xo1 = ((uint32_t)min(tok0 + 8 + lr, T - 1) * (uint32_t)d + 8u * lp) * 2u;
  const uint32_t wo = ((uint32_t)min(lane & 15, E - 1) * (uint32_t)d + 8u * (lane >> 4)) * 2u;
  // LDS: row r, logical piece q at r * 8 + (q ^ ((r >> 1) & 7))
  u32x4* t = tile[wave];
  const int wr0 = lr * 8 + (lp ^ ((lr >> 1) & 7));
  const int wr1 = (lr + 8) * 8 + (lp ^ (((lr + 8) >> 1) & 7));
  const int fr = lane & 15, fg = lane >> 4;
  const int rd0 = fr * 8 + ((fg) ^ ((fr >> 1) & 7));      // piece 0 * 4 + g
  const int rd1 = fr * 8 + ((4 + fg) ^ ((fr >> 1) & 7));  // piece 1 * 4 + g

  // Every k-pair issues exactly four loads (x rows 0-7, x rows 8-15, Wr for
  // MFMA 0, Wr for MFMA 1) for the pair P ahead -- past the end they re-read
  // the last pair -- so the wait for pair j leaves the 4 (P - 1) younger
  // loads in flight.  Asm loads with explicit waits: compiler-placed waits
  // drained the counter at every loop iteration.
  u32x4 xa[P], xb[P], w0[P], w1[P];
  auto issue = [&](int i, int j) {
    xa[i] = rload_async_nt(xs, xo0, j * 128);
    xb[i] = rload_async_nt(xs, xo1, j * 128);
    w0[i] = rload_async(ws, wo, j * 128);
    w1[i] = rload_async(ws, wo, j * 128 + 64);
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto consume = [&](int i) {
    t[wr0] = xa[i];
    t[wr1] = xb[i];
    const u32x4 b0 = t[rd0], b1 = t[rd1];
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w0[i]), as_bf16x8(b0), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w1[i]), as_bf16x8(b1), acc, 0, 0, 0);
  };
#pragma unroll
  for (int i = 0; i < P; ++i) issue(i, min(kb + i, ke - 1));
  int j0 = kb;
  for (; j0 + P <= ke; j0 += P) {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      rwait4<4 * P - 4>(xa[i], xb[i], w0[i], w1[i]);
      consume(i);
      issue(i, min(j0 + i + P, ke - 1));
    }
  }
  // the last ke - j0 < P pairs are in slots 0 ..; nothing else is in flight after
#pragma unroll
  for (int i = 0; i < P; ++i) {
    rwait4<0>(xa[i], xb[i], w0[i], w1[i]);
    if (j0 + i < ke) consume(i);
  }
  // acc[i] = z[token tok0 + (lane & 15)][expert 4 (lane >> 4) + i]
  const int tok = tok0 + (lane & 15);
  if (tok < T) {
    float* drow = dst + ((size_t)blockIdx.y * T + tok) * E;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * (lane >> 4) + i;
      if (e < E) drow[e] = acc[i];
    }
  }
}

// Split-K factor: enough blocks to cover the CUs (twice for the skinny kernel,
// whose blocks are latency-bound streams).  Partial logits are summed by the
// top-k kernel in split order, so the logits stay bitwise reproducible.
int router_splits(const moe_config& c) {
  if (c.dtype != MOE_BF16 || c.T == 0) return 1;
  if (c.E <= 16) {
    const long tiles = div_up(c.T, 64);
    long s = (512 + tiles - 1) / tiles;
    if (s > kMaxSplits) s = kMaxSplits;
    if (s > c.d / 64) s = c.d / 64;  // at least one k-pair per split
    return (int)(s < 1 ? 1 : s);
  }
  const int nch = c.d / 64;
  const int ec = c.E <= 32 ? 32 : c.E <= 64 ? 64 : c.E <= 128 ? 128 : 256;
  const long tiles = (long)div_up(c.T, 64) * div_up(c.E, ec);
  // blocks to aim for: each split adds T x E fp32 partials that the top-k
  // kernel reads back (measured best: 256 for E <= 64, 512 for E = 256)
  const long target = c.E <= 64 ? 256 : 512;
  long s = (target + tiles - 1) / tiles;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s > nch) s = nch;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_router_gemm_bf16(const uint16_t* x, const uint16_t* wr, float* dst, int T, int d,
                                   int E, int splits, hipStream_t st) {
  if (E <= 16) {
    router_skinny_bf16_kernel<<<dim3(div_up(T, 64), splits), 256, 0, st>>>(x, wr, dst, T, d, E,
                                                                           splits);
    return hipGetLastError();
  }
  const int ec = E <= 32 ? 32 : E <= 64 ? 64 : E <= 128 ? 128 : 256;  // E > 16 here
  dim3 grid(div_up(T, 64), splits, div_up(E, ec));
  switch (ec) {
    case 32: router_gemm_bf16_kernel<32><<<grid, 256, 0, st>>>(x, wr, dst, T, d, E, splits); break;
    case 64: router_gemm_bf16_kernel<64><<<grid, 256, 0, st>>>(x, wr, dst, T, d, E, splits); break;
    case 128: router_gemm_bf16_kernel<128><<<grid, 256, 0, st>>>(x, wr, dst, T, d, E, splits); break;
    default: router_gemm_bf16_kernel<256><<<grid, 256, 0, st>>>(x, wr, dst, T, d, E, splits); break;
  }
  return hipGetLastError();
}

// ============================================================== gate GEMM f32
// Small fp32 problems: one thread per logit, sequential fp32 FMA over d.
__global__ void router_gemm_f32_kernel(const float* __restrict__ x, const float* __restrict__ wr,
                                       float* __restrict__ z, int T, int d, int E) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)T * E) return;
  const int t = (int)(i / E), e = (int)(i % E);
  const float* xr = x + (size_t)t * d;
  const float* wrow = wr + (size_t)e * d;
  float acc = 0.f;
  for (int j = 0; j < d; ++j) acc = fmaf(xr[j], wrow[j], acc);
  z[i] = acc;
}

hipError_t launch_router_gemm_f32(const float* x, const float* wr, float* dst, int T, int d, int E,
                                  hipStream_t st) {
  const long n = (long)T * E;
  router_gemm_f32_kernel<<<div_up(n, 256), 256, 0, st>>>(x, wr, dst, T, d, E);
  return hipGetLastError();
}

// ============================================================== top-k + gates
__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  const int lo = __shfl_xor((int)(uint32_t)v, m);
  const int hi = __shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

template <int LPT>
__device__ __forceinline__ unsigned long long seg_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = LPT / 2; o > 0; o >>= 1) {
    const unsigned long long w = shfl_xor_u64(v, o);
    v = w > v ? w : v;
  }
  return v;
}

template <int LPT>
__device__ __forceinline__ uint32_t seg_max_u32(uint32_t v) {
#pragma unroll
  for (int o = LPT / 2; o > 0; o >>= 1) {
    const uint32_t w = (uint32_t)__shfl_xor((int)v, o);
    v = w > v ? w : v;
  }
  return v;
}

template <int LPT>
__device__ __forceinline__ float seg_sum(float v) {
#pragma unroll
  for (int o = LPT / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float ord_key_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

constexpr int kMaxEPL = 16;  // E <= 1024 with 64 lanes per token

// EPL: scores per lane (ceil(E / LPT): 1 for E <= 64), so the code holds only
// the loops a layer of this size needs.
template <int LPT, int EPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ partial, int splits,
                                                   const float* __restrict__ bias,
                                                   float* __restrict__ logits_out,
                                                   int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w, int T, int E, int k,
                                                   int n_group, int topk_group, int presel,
                                                   int renorm) {
  constexpr int TPW = 64 / LPT;  // tokens per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane % LPT;
  const int t = (blockIdx.x * 4 + wave) * TPW + lane / LPT;
  const bool live = t < T;
  const int epl = (E + LPT - 1) / LPT;

  // scores s = z + b (one fp32 add), -0 -> +0; key32 = order-preserving bits
  uint32_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    key[i] = 0u;
    const int e = q + i * LPT;
    if (i < epl && e < E && live) {
      // every partial is loaded before the first add (one memory latency),
      // then summed in split order
      float pv[kMaxSplits];
#pragma unroll
      for (int s = 0; s < kMaxSplits; ++s)
        pv[s] = s < splits ? partial[((size_t)s * T + t) * E + e] : 0.f;
      float z = pv[0];
#pragma unroll
      for (int s = 1; s < kMaxSplits; ++s)
        if (s < splits) z += pv[s];
      if (logits_out) logits_out[(size_t)t * E + e] = z;
      float sc = bias ? __fadd_rn(z, bias[e]) : z;
      uint32_t u = __float_as_uint(sc);
      if (u == 0x80000000u) u = 0u;
      key[i] = ord_key(__uint_as_float(u));
    }
  }

  // group-limited eligibility: keep the topk_group groups with the largest max
  unsigned long long kept = ~0ull;
  const bool grouped = n_group > 1 && topk_group < n_group;
  int gsz = E / n_group;
  if (grouped) {
    uint32_t my_g = 0u;
    for (int g = 0; g < n_group; ++g) {
      uint32_t m = 0u;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = q + i * LPT;
        if (i < epl && e < E && e / gsz == g) m = key[i] > m ? key[i] : m;
      }
      m = seg_max_u32<LPT>(m);
      if (q == g) my_g = m;
    }
    kept = 0ull;
    for (int r = 0; r < topk_group; ++r) {
      unsigned long long cand = 0ull;
      if (q < n_group && !((kept >> q) & 1ull))
        cand = ((unsigned long long)my_g << 32) | (0xffffffffu - (uint32_t)q);
      cand = seg_max_u64<LPT>(cand);
      const int gw = (int)(0xffffffffu - (uint32_t)cand);
      kept |= 1ull << gw;
    }
  }

  // selection rounds: the r-th winner is kept by lane q == r
  const int nsel = presel > k ? presel : k;
  uint32_t taken = 0u;
  int my_e = 0;
  float my_s = 0.f, s_max = 0.f;
  for (int r = 0; r < nsel; ++r) {
    unsigned long long best = 0ull;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = q + i * LPT;
      const bool ok = i < epl && e < E && !((taken >> i) & 1u) &&
                      (!grouped || ((kept >> (e / gsz)) & 1ull));
      const unsigned long long cand =
          ok ? (((unsigned long long)key[i] << 32) | (0xffffffffu - (uint32_t)e)) : 0ull;
      best = cand > best ? cand : best;
    }
    best = seg_max_u64<LPT>(best);
    const int we = (int)(0xffffffffu - (uint32_t)best);
    const float ws = ord_key_inv((uint32_t)(best >> 32));
    if (we % LPT == q) taken |= 1u << (we / LPT);
    if (r == 0) s_max = ws;
    if (q == r) {
      my_e = we;
      my_s = ws;
    }
  }

  // gates: e_j = exp(s_j - m) over the chosen / pre-selected / all experts
  const float ej = q < nsel ? expf(my_s - s_max) : 0.f;
  float denom;
  if (renorm) {
    denom = seg_sum<LPT>(q < k ? ej : 0.f);
  } else if (presel) {
    denom = seg_sum<LPT>(q < presel ? ej : 0.f);
  } else {
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = q + i * LPT;
      if (i < epl && e < E) part += expf(ord_key_inv(key[i]) - s_max);
    }
    denom = seg_sum<LPT>(part);
  }
  if (live && q < k) {
    topk_idx[(size_t)t * k + q] = my_e;
    topk_w[(size_t)t * k + q] = ej / denom;
  }
}

hipError_t launch_topk(const moe_config& c, const float* partial, int splits, const float* bias,
                       float* logits_out, int32_t* topk_idx, float* topk_w, hipStream_t st) {
  if (splits < 1 || splits > kMaxSplits) return hipErrorInvalidValue;
  int lpt = 1;
  while (lpt < c.E && lpt < 64) lpt <<= 1;
  if (lpt < 2) lpt = 2;
  // 64 < E <= 256: 32 lanes of 8 scores each, two tokens per wave (fewer
  // shuffle steps per selection round; E=256: 97 -> 92 us for T=8192).  The
  // group maxima sit one per lane, so this needs n_group <= 32.
  if (c.E > 64 && c.E <= 256 && c.n_group <= 32) lpt = 32;
  const int tpb = 4 * (64 / lpt);
  const dim3 grid(div_up(c.T, tpb));
#define MOE_TOPK(L, P)                                                                        \
  topk_kernel<L, P><<<grid, 256, 0, st>>>(partial, splits, bias, logits_out, topk_idx, topk_w, \
                                          c.T, c.E, c.k, c.n_group, c.topk_group, c.presel,    \
                                          c.renorm)
  switch (lpt) {
    case 2: MOE_TOPK(2, 1); break;
    case 4: MOE_TOPK(4, 1); break;
    case 8: MOE_TOPK(8, 1); break;
    case 16: MOE_TOPK(16, 1); break;
    case 32:
      if (c.E > 64)
        MOE_TOPK(32, 8);
      else
        MOE_TOPK(32, 1);
      break;
    default:
      if (c.E <= 64)
        MOE_TOPK(64, 1);
      else
        MOE_TOPK(64, kMaxEPL);
      break;
  }
#undef MOE_TOPK
  return hipGetLastError();
}

}  // namespace moe
