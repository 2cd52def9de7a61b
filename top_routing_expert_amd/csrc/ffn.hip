// Grouped expert FFN: for each expert e, rows [off[e], off[e+1]) of the
// permuted activations go through  h = SiLU(X Wg^T) * (X Wu^T)  (gate_up) and
// y = h Wd^T  (down).
//
// Pages: [V4-overlap] Waved-EP section (expert compute = L1 + Act + L2);
// [EP-V4] §5.2 (expert weights contiguous and in expert-ID order, which is
// what lets neighbouring tiles share weight lines in cache); [SyncTax] §2.2
// (skewed expert load: hot experts must not stall the rest).
//
// gfx950 design (one kernel template, two instantiations)
//  * Tile = 256 weight rows x 128 token rows x 64 k.  The weights are the MFMA
//    A operand (M side) and the tokens the B operand (N side), so each lane's
//    four accumulator values are four consecutive OUTPUT FEATURES of one token
//    and the epilogue stores 8 contiguous bytes per lane.
//    gate_up: the 256 weight rows are 128 rows of W_gate and the same 128 rows
//    of W_up, so each wave holds matching gate/up accumulators and applies
//    SiLU(g)*u in registers (no extra pass over h).  down: 256 rows of W_down.
//  * 4 waves in a 2 (weights) x 2 (tokens) layout, 128 fp32 accumulators per
//    lane; MFMA f32_16x16x32_bf16, 64 MFMAs per wave per k step.
//  * Global -> register prefetch of the next k step while the current one is
//    multiplied out of LDS; two LDS stages (96 KB), one barrier per k step.
//    LDS rows are 128 B; 16-byte pieces are XOR-swizzled with (row & 7) so the
//    fragment reads of 8 consecutive rows hit distinct banks.
//  * No host sync: the row table is read on the device.  Each block rebuilds
//    the per-expert tile prefix sum from expert_offsets with one wave, finds
//    its (expert, row tile) and exits if it has none; the grid is sized for
//    the worst case  sum_e ceil(c_e/128) <= (rows + E*127)/128.  Skewed
//    experts therefore just own more tiles.
//  * Rasterisation: tiles are ordered expert by expert; inside an expert in
//    bands of up to 8 row tiles, and inside a band by weight tile with the row
//    tiles fastest.  The tiles that run at the same time on one XCD therefore
//    share one expert's weight rows (across row tiles) and token rows (across
//    weight tiles) in that XCD's L2.  The device-side tile count is dealt to
//    the 8 XCDs (blocks are dispatched to XCDs round-robin) in equal
//    contiguous ranges, so the empty slots of the worst-case grid never pile
//    up on one XCD.
#include "common.h"

namespace moe {

constexpr int BM = kGemmBM;    // 128 token rows
constexpr int BNW = kGemmBNW;  // 256 weight rows
constexpr int BK = kGemmBK;    // 64

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const lds_void_t*)p;
}

// Direct global -> LDS copy of 16 bytes per lane: lane L of the issuing wave
// writes LDS bytes [lds + 16 L, lds + 16 L + 16); `lds` is wave-uniform.  Issued
// as inline asm so that the wait for it stays under this kernel's explicit
// vmcnt control (the compiler would otherwise drain every copy in flight
// before each LDS read).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N of this wave's vector-memory operations are in flight,
// then barrier.  No memory fence: the LDS DMA traffic is ordered by vmcnt.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

constexpr int kStages = 3;
constexpr int kChunksA = BNW * 128 / 1024;         // 1 KB LDS chunks per stage: 32 weights
constexpr int kChunksB = BM * 128 / 1024;          // 16 tokens
constexpr int kDmaPerWave = (kChunksA + kChunksB) / 4;  // 12

template <bool GATED>
__global__ __launch_bounds__(256, 1) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ offs,
    const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1, uint16_t* __restrict__ out,
    int E, int N, int K, int rows, int n_tiles, int band) {
  // per stage: weights 256 rows x 128 B, then tokens 128 rows x 128 B
  __shared__ u32x4 sbuf[kStages][(kChunksA + kChunksB) * 64];
  __shared__ int s_tile[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- which tile: one wave reads the row table and places this block.
  // Tiles are ordered expert by expert; inside an expert, in bands of up to
  // `band` row tiles, and inside a band by weight tile with the row tiles
  // fastest.  The actual tile count (known only on the device) is dealt to
  // the 8 XCDs in equal contiguous ranges (blocks go to XCDs round-robin), so
  // the tiles running at once on one XCD share weight and token rows in L2
  // and no XCD is left with only empty slots.
  if (wave == 0) {
    if (lane == 0) s_tile[0] = -1;
    int total = 0;
    for (int b0 = 0; b0 < E; b0 += 64) {
      const int e = b0 + lane;
      int nt = 0;
      if (e < E) {  // clamp a malformed table into [0, rows] so accesses stay in bounds
        const int o0 = min(max(offs[e], 0), rows), o1 = min(max(offs[e + 1], o0), rows);
        nt = (o1 - o0 + BM - 1) / BM;
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) nt += __shfl_xor(nt, o);
      total += nt;
    }
    const int n_total = total * n_tiles;
    const int per_xcd = (n_total + 7) >> 3;
    const int L = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if ((int)(blockIdx.x >> 3) < per_xcd && L < n_total) {
      int carry = 0;  // tiles of the experts before this 64-expert chunk
      for (int b0 = 0; b0 < E; b0 += 64) {
        const int e = b0 + lane;
        int o0 = 0, o1 = 0;
        if (e < E) {
          o0 = min(max(offs[e], 0), rows);
          o1 = min(max(offs[e + 1], o0), rows);
        }
        const int mt = (o1 - o0 + BM - 1) / BM;
        int incl = mt * n_tiles;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o);
          if (lane >= o) incl += y;
        }
        const int excl = carry + incl - mt * n_tiles;
        if (mt > 0 && L >= excl && L < excl + mt * n_tiles) {
          const int r = L - excl;
          const int g = min(band, mt);
          const int full = mt / g;
          int n, m;
          if (r < full * g * n_tiles) {
            const int bi = r / (g * n_tiles), rr = r - bi * g * n_tiles;
            n = rr / g;
            m = bi * g + rr % g;
          } else {
            const int gl = mt - full * g, rr = r - full * g * n_tiles;
            n = rr / gl;
            m = full * g + rr % gl;
          }
          s_tile[0] = e;
          s_tile[1] = o0 + m * BM;
          s_tile[2] = o1;
          s_tile[3] = n;
        }
        carry += __shfl(incl, 63);
      }
    }
  }
  __syncthreads();
  const int e = s_tile[0];
  if (e < 0) return;  // block-uniform
  const int row0 = s_tile[1], row_end = s_tile[2], n_tile = s_tile[3];
  const int n0 = n_tile * (GATED ? BNW / 2 : BNW);

  // ---- DMA assignment.  Wave w copies LDS chunks c = w + 4 i (i < 12) of every
  // stage; chunk c < 32 holds weight-tile rows 8c..8c+7, the others token-tile
  // rows.  Lane l lands at row 8c' + l/8, physical 16-byte piece l%8, so it
  // fetches the logical piece (l%8) ^ (row & 7) = (l & 7) ^ (l >> 3): the LDS
  // image is XOR-swizzled exactly as the fragment reads below expect.
  const int lr = lane >> 3;
  const int lq = (lane & 7) ^ lr;
  const uint16_t* gsrc[kDmaPerWave];
  int ldst[kDmaPerWave];  // u32x4 index of the chunk inside a stage
  const size_t wstride = (size_t)N * K;
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int c = wave + 4 * i;
    ldst[i] = c * 64;
    if (c < kChunksA) {
      const int r = 8 * c + lr;  // weight tile row 0..255
      const uint16_t* base;
      int n;
      if (GATED) {
        n = n0 + (r & 127);
        base = (r < 128 ? w0 : w1) + (size_t)e * wstride;
      } else {
        n = n0 + r;
        base = w0 + (size_t)e * wstride;
      }
      n = min(n, N - 1);
      gsrc[i] = base + (size_t)n * K + lq * 8;
    } else {
      const int r = min(row0 + 8 * (c - kChunksA) + lr, row_end - 1);
      gsrc[i] = act + (size_t)r * K + lq * 8;
    }
  }

  // ---- fragment addressing (constant per lane)
  const int wn = wave >> 1, wm = wave & 1;
  int arow[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (GATED)
      arow[i] = (i < 4 ? 0 : 128) + wn * 64 + (i & 3) * 16 + (lane & 15);
    else
      arow[i] = wn * 128 + i * 16 + (lane & 15);
  }
  int brow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) brow[j] = BNW + wm * 64 + j * 16 + (lane & 15);  // token rows follow
  const int lsw = lane & 7;  // (row & 7) of every fragment row this lane reads

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK;
  const uint32_t lds0 = lds_addr(&sbuf[0][0]);
  auto issue = [&](int kt, int st) {
    const uint32_t sbase = lds0 + (uint32_t)st * (kChunksA + kChunksB) * 1024u;
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i)
      dma16(gsrc[i] + (size_t)kt * BK, sbase + (uint32_t)ldst[i] * 16u);
  };
  issue(0, 0);
  if (nk > 1) issue(1, 1);

  int st = 0;
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's copies of stage kt are done once only stage kt+1's (if any)
    // remain in flight; the barrier then publishes every wave's copies and
    // guarantees that nobody still reads the buffer refilled below
    if (kt + 1 < nk)
      wait_vm_barrier<kDmaPerWave>();
    else
      wait_vm_barrier<0>();
    if (kt + 2 < nk) issue(kt + 2, st == 0 ? 2 : st - 1);
    const u32x4* sb = sbuf[st];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int q = (4 * s + (lane >> 4)) ^ lsw;
      bf16x8 a[8], b[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] = as_bf16x8(sb[arow[i] * 8 + q]);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = as_bf16x8(sb[brow[j] * 8 + q]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    st = st == 2 ? 0 : st + 1;
  }

  // ---- epilogue: acc[i][j][r] = C[weight row arow_base(i) + 4(lane>>4) + r][token brow[j]]
  const int g4 = 4 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = row0 + brow[j] - BNW;
    if (row >= row_end) continue;
    uint16_t* orow = out + (size_t)row * N;
    if (GATED) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + wn * 64 + i * 16 + g4;
        if (n >= N) continue;
        float hv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gt = acc[i][j][r], up = acc[i + 4][j][r];
          hv[r] = gt / (1.0f + __expf(-gt)) * up;
        }
        u32x2 pk;
        pk.x = pack_bf16x2(hv[0], hv[1]);
        pk.y = pack_bf16x2(hv[2], hv[3]);
        *reinterpret_cast<u32x2*>(orow + n) = pk;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int n = n0 + wn * 128 + i * 16 + g4;
        if (n >= N) continue;
        u32x2 pk;
        pk.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
        pk.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        *reinterpret_cast<u32x2*>(orow + n) = pk;
      }
    }
  }
}

// ------------------------------------------------------------------ fp32 path
// Small fp32 problems: one thread per output element, sequential fp32 FMA.
__device__ __forceinline__ int expert_of_row(const int32_t* offs, int E, int p) {
  int lo = 0, hi = E;  // largest e with offs[e] <= p, among e in [0, E)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offs[mid] <= p) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ void ffn_gate_up_f32_kernel(const float* __restrict__ xp, const int32_t* __restrict__ offs,
                                       const float* __restrict__ wg, const float* __restrict__ wu,
                                       float* __restrict__ h, int E, int f, int d, long rows) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long r0 = min(max(offs[0], 0), (int)rows), r1 = min(max(offs[E], 0), (int)rows);
  const long p = r0 + i / f;
  if (i >= rows * f || p >= r1) return;
  const int n = (int)(i % f);
  const int e = expert_of_row(offs, E, (int)p);
  const float* xr = xp + p * d;
  const float* g = wg + ((size_t)e * f + n) * d;
  const float* u = wu + ((size_t)e * f + n) * d;
  float a = 0.f, b = 0.f;
  for (int j = 0; j < d; ++j) {
    a = fmaf(xr[j], g[j], a);
    b = fmaf(xr[j], u[j], b);
  }
  h[p * f + n] = a / (1.0f + expf(-a)) * b;
}

__global__ void ffn_down_f32_kernel(const float* __restrict__ h, const int32_t* __restrict__ offs,
                                    const float* __restrict__ wd, float* __restrict__ y, int E, int d,
                                    int f, long rows) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long r0 = min(max(offs[0], 0), (int)rows), r1 = min(max(offs[E], 0), (int)rows);
  const long p = r0 + i / d;
  if (i >= rows * d || p >= r1) return;
  const int n = (int)(i % d);
  const int e = expert_of_row(offs, E, (int)p);
  const float* hr = h + p * f;
  const float* w = wd + ((size_t)e * d + n) * f;
  float a = 0.f;
  for (int j = 0; j < f; ++j) a = fmaf(hr[j], w[j], a);
  y[p * d + n] = a;
}

// ------------------------------------------------------------------ launchers
static void gemm_grid(int rows, int E, int N_out_per_tile, int N, int* n_tiles, int* band,
                      int* blocks) {
  *n_tiles = div_up(N, N_out_per_tile);
  // upper bound of sum_e ceil(c_e / BM) over any row table with `rows` rows
  long m_slots = ((long)rows + (long)E * (BM - 1)) / BM;
  if (m_slots < 1) m_slots = 1;
  *band = 8;
  const long total = (long)(*n_tiles) * m_slots;
  *blocks = (int)((total + 7) / 8 * 8);
}

hipError_t launch_ffn_gate_up(const moe_config& c, const void* x_perm, const int32_t* offs,
                              const void* wg, const void* wu, void* h, hipStream_t st) {
  const long rows = (long)c.T * c.k;
  if (c.dtype == MOE_F32) {
    const long n = rows * c.f;
    ffn_gate_up_f32_kernel<<<div_up(n, 256), 256, 0, st>>>(
        static_cast<const float*>(x_perm), offs, static_cast<const float*>(wg),
        static_cast<const float*>(wu), static_cast<float*>(h), c.E, c.f, c.d, rows);
    return hipGetLastError();
  }
  int n_tiles, band, blocks;
  gemm_grid((int)rows, c.E, BNW / 2, c.f, &n_tiles, &band, &blocks);
  grouped_gemm_bf16_kernel<true><<<blocks, 256, 0, st>>>(
      static_cast<const uint16_t*>(x_perm), offs, static_cast<const uint16_t*>(wg),
      static_cast<const uint16_t*>(wu), static_cast<uint16_t*>(h), c.E, c.f, c.d, (int)rows,
      n_tiles, band);
  return hipGetLastError();
}

hipError_t launch_ffn_down(const moe_config& c, const void* h, const int32_t* offs, const void* wd,
                           void* y, hipStream_t st) {
  const long rows = (long)c.T * c.k;
  if (c.dtype == MOE_F32) {
    const long n = rows * c.d;
    ffn_down_f32_kernel<<<div_up(n, 256), 256, 0, st>>>(
        static_cast<const float*>(h), offs, static_cast<const float*>(wd), static_cast<float*>(y),
        c.E, c.d, c.f, rows);
    return hipGetLastError();
  }
  int n_tiles, band, blocks;
  gemm_grid((int)rows, c.E, BNW, c.d, &n_tiles, &band, &blocks);
  grouped_gemm_bf16_kernel<false><<<blocks, 256, 0, st>>>(
      static_cast<const uint16_t*>(h), offs, static_cast<const uint16_t*>(wd), nullptr,
      static_cast<uint16_t*>(y), c.E, c.d, c.f, (int)rows, n_tiles, band);
  return hipGetLastError();
}

}  // namespace moe
