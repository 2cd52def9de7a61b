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
//  * Rasterisation: tiles are ordered in bands of `band` row tiles; inside a
//    band all weight tiles (n) are visited with the row tiles fastest, so the
//    tiles that share one expert's weight rows run back to back, and the
//    band's token rows stay cache resident.  Block ids are remapped so that
//    each XCD (blocks are dealt round-robin to the 8 XCDs) walks one
//    contiguous range of that order and keeps its L2 working set local.
#include "common.h"

namespace moe {

constexpr int BM = kGemmBM;    // 128 token rows
constexpr int BNW = kGemmBNW;  // 256 weight rows
constexpr int BK = kGemmBK;    // 64

template <bool GATED>
__global__ __launch_bounds__(256, 1) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ offs,
    const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1, uint16_t* __restrict__ out,
    int E, int N, int K, int rows, int n_tiles, int m_slots, int band) {
  __shared__ u32x4 sA[2][BNW * 8];  // weights: 256 rows x 128 B
  __shared__ u32x4 sB[2][BM * 8];   // tokens : 128 rows x 128 B
  __shared__ int s_tile[3];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // ---- logical tile: XCD-contiguous remap, then bands of row tiles
  const int nb = gridDim.x;  // multiple of 8
  const int L = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
  if (L >= n_tiles * m_slots) return;
  const int per_band = band * n_tiles;
  const int bi = L / per_band;
  const int rr = L - bi * per_band;
  const int mb = min(band, m_slots - bi * band);
  const int n_tile = rr / mb;
  const int m_slot = bi * band + rr % mb;

  // ---- find (expert, row range) of row-tile slot m_slot on the device
  if (wave == 0) {
    if (lane == 0) s_tile[0] = -1;
    int carry = 0;
    for (int b0 = 0; b0 < E; b0 += 64) {
      const int e = b0 + lane;
      int o0 = 0, o1 = 0;
      if (e < E) {  // clamp a malformed table into [0, rows] so accesses stay in bounds
        o0 = min(max(offs[e], 0), rows);
        o1 = min(max(offs[e + 1], o0), rows);
      }
      const int nt = o1 > o0 ? (o1 - o0 + BM - 1) / BM : 0;
      int incl = nt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      const int excl = carry + incl - nt;
      if (nt > 0 && m_slot >= excl && m_slot < excl + nt) {
        s_tile[0] = e;
        s_tile[1] = o0 + (m_slot - excl) * BM;
        s_tile[2] = o1;
      }
      carry += __shfl(incl, 63);
    }
  }
  __syncthreads();
  const int e = s_tile[0];
  if (e < 0) return;  // block-uniform
  const int row0 = s_tile[1], row_end = s_tile[2];
  const int n0 = n_tile * (GATED ? BNW / 2 : BNW);

  // ---- global load assignment: 8 threads per 128-byte row piece
  const int lrow = tid >> 3, lq = tid & 7;
  const u32x4* gA[8];
  const u32x4* gB[4];
  const size_t wstride = (size_t)N * K;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = lrow + 32 * i;  // weight tile row 0..255
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
    gA[i] = reinterpret_cast<const u32x4*>(base + (size_t)n * K) + lq;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = min(row0 + lrow + 32 * i, row_end - 1);
    gB[i] = reinterpret_cast<const u32x4*>(act + (size_t)r * K) + lq;
  }
  const int sw = lq ^ (lrow & 7);  // (lrow + 32 i) & 7 == lrow & 7

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
  for (int j = 0; j < 4; ++j) brow[j] = wm * 64 + j * 16 + (lane & 15);
  const int lsw = lane & 7;  // (row & 7) of every fragment row this lane reads

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[8], rb[4];
  const int nk = K / BK;
#pragma unroll
  for (int i = 0; i < 8; ++i) ra[i] = gA[i][0];
#pragma unroll
  for (int i = 0; i < 4; ++i) rb[i] = gB[i][0];
#pragma unroll
  for (int i = 0; i < 8; ++i) sA[0][(lrow + 32 * i) * 8 + sw] = ra[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) sB[0][(lrow + 32 * i) * 8 + sw] = rb[i];
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int koff = (kt + 1) * 8;  // u32x4 units
#pragma unroll
      for (int i = 0; i < 8; ++i) ra[i] = gA[i][koff];
#pragma unroll
      for (int i = 0; i < 4; ++i) rb[i] = gB[i][koff];
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int q = (4 * s + (lane >> 4)) ^ lsw;
      bf16x8 a[8], b[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] = as_bf16x8(sA[st][arow[i] * 8 + q]);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = as_bf16x8(sB[st][brow[j] * 8 + q]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < 8; ++i) sA[st ^ 1][(lrow + 32 * i) * 8 + sw] = ra[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) sB[st ^ 1][(lrow + 32 * i) * 8 + sw] = rb[i];
    }
    __syncthreads();
  }

  // ---- epilogue: acc[i][j][r] = C[weight row arow_base(i) + 4(lane>>4) + r][token brow[j]]
  const int g4 = 4 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = row0 + brow[j];
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
static void gemm_grid(int rows, int E, int N_out_per_tile, int N, int K, int* n_tiles, int* m_slots,
                      int* band, int* blocks) {
  *n_tiles = div_up(N, N_out_per_tile);
  *m_slots = (int)(((long)rows + (long)E * (BM - 1)) / BM);
  if (*m_slots < 1) *m_slots = 1;
  // keep a band's token rows (band * BM * K * 2 bytes) around 48 MB
  long b = (48l << 20) / ((long)BM * K * 2);
  if (b < 1) b = 1;
  if (b > *m_slots) b = *m_slots;
  *band = (int)b;
  const long total = (long)(*n_tiles) * (*m_slots);
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
  int n_tiles, m_slots, band, blocks;
  gemm_grid((int)rows, c.E, BNW / 2, c.f, c.d, &n_tiles, &m_slots, &band, &blocks);
  grouped_gemm_bf16_kernel<true><<<blocks, 256, 0, st>>>(
      static_cast<const uint16_t*>(x_perm), offs, static_cast<const uint16_t*>(wg),
      static_cast<const uint16_t*>(wu), static_cast<uint16_t*>(h), c.E, c.f, c.d, (int)rows,
      n_tiles, m_slots, band);
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
  int n_tiles, m_slots, band, blocks;
  gemm_grid((int)rows, c.E, BNW, c.d, c.f, &n_tiles, &m_slots, &band, &blocks);
  grouped_gemm_bf16_kernel<false><<<blocks, 256, 0, st>>>(
      static_cast<const uint16_t*>(h), offs, static_cast<const uint16_t*>(wd), nullptr,
      static_cast<uint16_t*>(y), c.E, c.d, c.f, (int)rows, n_tiles, m_slots, band);
  return hipGetLastError();
}

}  // namespace moe
