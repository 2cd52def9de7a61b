// Grouped expert FFN: for each expert e, rows [off[e], off[e+1]) of the
// permuted activations go through  h = SiLU(X Wg^T) * (X Wu^T)  (gate_up) and
// y = h Wd^T  (down).
//
// Pages: [V4-overlap] Waved-EP section (expert compute = L1 + Act + L2);
// [EP-V4] §5.2 (expert weights contiguous and in expert-ID order, which is
// what lets neighbouring tiles share weight lines in cache); [SyncTax] §2.2
// (skewed expert load: hot experts must not stall the rest).
//
// gfx950 design
//  * Weights are the MFMA A operand (M side), tokens the B operand (N side),
//    so each lane's accumulator groups hold four consecutive OUTPUT FEATURES
//    of one token and the epilogue stores 8 contiguous bytes per lane.
//    gate_up: a tile's weight rows are rows n0.. of W_gate followed by the
//    same rows of W_up, so every wave holds matching gate/up accumulators and
//    applies SiLU(g)*u in registers (no extra pass over h).
//  * MFMA f32_32x32x16_bf16 (a single wave per SIMD keeps this instruction at
//    full rate; the 16x16x32 form needs two).  Four waves in a 2 (weights) x
//    2 (tokens) layout.  Two tile shapes: 256 weight rows x 256 tokens (128 x
//    128 per wave, 256 accumulators, one block per CU) for many rows per
//    expert, and 256 x 128 (128 accumulators, two blocks per CU so one block's
//    MFMAs overlap the other's memory phases) otherwise.
//  * Operands reach LDS through the gfx950 LDS-DMA load
//    (global_load_lds_dwordx4): no staging registers, 16 bytes per lane, each
//    wave instruction fills eight full 128-byte lines.  32-wide k stages in a
//    ring of 4 (or 3) buffers, several stages in flight, explicit vmcnt waits
//    and one barrier per stage.  LDS rows are 64 bytes; 16-byte pieces are
//    XOR-swizzled with (row >> 2) & 3, the pattern that measured fastest for
//    the 32-row fragment reads.
//  * The next stage's fragments are read from LDS while the current stage's
//    MFMAs run (two register sets, 2x unrolled k loop), so LDS reads overlap
//    matrix work instead of bunching after each barrier.
//  * Token fragments past the expert's last row skip their LDS reads and
//    MFMAs (the main loop is specialised on the live fragment count).
//  * No host sync: the row table is read on the device.  Each block rebuilds
//    the per-expert tile prefix sum from expert_offsets with one wave, finds
//    its (expert, row tile) and exits if it has none; the grid is sized for
//    the worst case  sum_e ceil(c_e/TM) <= (rows + E*(TM-1))/TM.  Skewed
//    experts therefore just own more tiles.
//  * Rasterisation: tiles are ordered expert by expert; inside an expert in
//    bands of up to 8 row tiles, and inside a band by weight tile with the row
//    tiles fastest.  The tiles that run at the same time on one XCD therefore
//    share one expert's weight rows (across row tiles) and token rows (across
//    weight tiles) in that XCD's L2.  The device-side tile count is dealt to
//    the 8 XCDs (blocks are dispatched to XCDs round-robin) in equal
//    contiguous ranges, so the empty slots of the worst-case grid never pile
//    up on one XCD.
#include <type_traits>

#include "common.h"
#include "tiles.h"

namespace moe {

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const lds_void_t*)p;
}

// Direct global -> LDS copy of 16 bytes per lane: lane L of the issuing wave
// writes LDS bytes [lds + 16 L, lds + 16 L + 16); `lds` is wave-uniform.  Issued
// as inline asm so that the wait for it stays under this kernel's explicit
// vmcnt control (the compiler would otherwise drain every copy in flight
// before each LDS read).  The kernel issues no other vector-memory reads in
// its main loop, so the counts below are exact.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory operations are in flight,
// then barrier.  No memory fence: the LDS DMA traffic is ordered by vmcnt.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// LDS image of one stage: rows of 64 bytes (32 k), weight-tile rows first,
// then token-tile rows; the 16-byte piece q of row r sits at q ^ ((r >> 2) & 3).
__device__ __forceinline__ int lds_piece(int r, int q) { return r * 4 + (q ^ ((r >> 2) & 3)); }

constexpr int kStages = 4;
constexpr int kStageK = 32;

// WA / WB: 32-row fragments per wave on the weight / token side.  Four waves
// in a 2 (weights) x 2 (tokens) layout; the block tile is 64 WA weight rows
// by 64 WB token rows.
template <bool GATED, int WA, int WB>
__global__ __launch_bounds__(256, (WB == 2 ? 2 : 1)) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ offs,
    const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1, uint16_t* __restrict__ out,
    int E, int N, int K, int rows, int n_tiles, int band) {
  constexpr int TW = 64 * WA;                   // weight rows per tile
  constexpr int TM = 64 * WB;                   // token rows per tile
  constexpr int TN = GATED ? TW / 2 : TW;       // output features per tile
  constexpr int ROWS = TW + TM;                 // LDS rows per stage
  constexpr int CHUNKS = ROWS * 64 / 1024;      // 1 KB DMA chunks per stage
  constexpr int DPW = CHUNKS / 4;               // DMA instructions per wave per stage
  constexpr int STAGES = WB == 2 ? 3 : kStages;  // LDS ring depth (two 128-token blocks per CU)
  static_assert(CHUNKS % 4 == 0, "stage must split evenly over 4 waves");
  static_assert(STAGES * ROWS * 64 <= 150 * 1024, "LDS ring too large");
  __shared__ u32x4 sbuf[STAGES][ROWS * 4];
  __shared__ int s_tile[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- which tile (one wave reads the row table)
  if (wave == 0) place_tile<TM>(offs, E, rows, n_tiles, band, lane, s_tile);
  __syncthreads();
  const int e = s_tile[0];
  if (e < 0) return;  // block-uniform
  const int row0 = s_tile[1], row_end = s_tile[2], n_tile = s_tile[3];
  const int n0 = n_tile * TN;
  const int nk = K / kStageK;
  const size_t wstride = (size_t)N * K;

  // ---- DMA assignment.  Wave w copies chunks c = w + 4 i (i < DPW) of every
  // stage; chunk c holds LDS rows 16c..16c+15 (weight rows first).  Lane l
  // lands at row 16c + l/4, physical piece l%4, so it fetches the logical
  // piece (l & 3) ^ ((row >> 2) & 3) = (l & 3) ^ ((l >> 4) & 3).
  const int lq = (lane & 3) ^ ((lane >> 4) & 3);
  const uint16_t* gsrc[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int r = 16 * (wave + 4 * i) + (lane >> 2);  // LDS row 0..ROWS-1
    if (r < TW) {
      const uint16_t* base;
      int n;
      if (GATED) {
        n = n0 + (r % (TW / 2));
        base = (r < TW / 2 ? w0 : w1) + (size_t)e * wstride;
      } else {
        n = n0 + r;
        base = w0 + (size_t)e * wstride;
      }
      n = min(n, N - 1);
      gsrc[i] = base + (size_t)n * K + lq * 8;
    } else {
      const int t = min(row0 + (r - TW), row_end - 1);
      gsrc[i] = act + (size_t)t * K + lq * 8;
    }
  }

  // ---- fragments.  MFMA 32x32x16: lane l holds row (l & 31) of a 32-row
  // fragment and k in [8 (l >> 5), 8 (l >> 5) + 8) of a 16-wide slab, for
  // weights (A) and tokens (B) alike.  Wave (wn, wm) owns WA weight fragments
  // (GATED: WA/2 gate fragments and the matching up fragments, i.e. 32 WA/2
  // output features) and WB token fragments.
  const int wn = wave >> 1, wm = wave & 1;
  const int lk = lane >> 5;
  int arow[WA];
#pragma unroll
  for (int i = 0; i < WA; ++i) {
    if (GATED)
      arow[i] = (i < WA / 2 ? 0 : TW / 2) + wn * 16 * WA + (i % (WA / 2)) * 32 + (lane & 31);
    else
      arow[i] = wn * 32 * WA + i * 32 + (lane & 31);
  }
  // token fragments of this wave that hold any row; the others are skipped
  const int tok0 = wm * 32 * WB;
  const int jn = __builtin_amdgcn_readfirstlane(min(WB, max(0, (row_end - row0 - tok0 + 31) >> 5)));
  const int brow0 = TW + tok0 + (lane & 31);

  f32x16 acc[WA][WB];
#pragma unroll
  for (int i = 0; i < WA; ++i)
#pragma unroll
    for (int j = 0; j < WB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const uint32_t lds0 = lds_addr(&sbuf[0][0]);
  auto issue = [&](int kt) {
    const uint32_t sbase = lds0 + (uint32_t)(kt % STAGES) * (ROWS * 64u);
#pragma unroll
    for (int i = 0; i < DPW; ++i)
      dma16(gsrc[i] + (size_t)kt * kStageK, sbase + (uint32_t)(wave + 4 * i) * 1024u);
  };
  // Main loop, specialised on JN = token fragments of this wave that hold any
  // row (wave-uniform; the other fragments' reads and MFMAs are skipped).
  auto main_loop = [&](auto jn_c) {
    constexpr int JN = decltype(jn_c)::value;
    // fragments of one 32-wide stage: two 16-wide slabs
    struct Frags {
      bf16x8 a[2][WA];
      bf16x8 b[2][WB];
    };
    auto load_frags = [&](int kt, Frags& F) {
      const u32x4* sb = sbuf[kt % STAGES];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int q = 2 * s2 + lk;
#pragma unroll
        for (int i = 0; i < WA; ++i) F.a[s2][i] = as_bf16x8(sb[lds_piece(arow[i], q)]);
#pragma unroll
        for (int j = 0; j < JN; ++j) F.b[s2][j] = as_bf16x8(sb[lds_piece(brow0 + 32 * j, q)]);
      }
    };
    auto mfma_stage = [&](const Frags& F) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int j = 0; j < JN; ++j)
#pragma unroll
          for (int i = 0; i < WA; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.a[s2][i], F.b[s2][j], acc[i][j],
                                                                0, 0, 0);
    };
    // Pipeline.  Stage j (32-wide k-step j) goes to LDS buffer j % STAGES.
    // Stage kt's fragments are read during step kt-1, while its MFMAs run, so
    // LDS reads overlap the matrix work instead of bunching after a barrier.
    // End of step kt: wait for this wave's copies of stage kt+2, barrier (all
    // copies of kt+2 visible; nobody reads stages kt, kt+1 any more), then
    // refill buffer kt % STAGES with stage kt + STAGES.
    auto wait_for = [&](int j) {  // own copies of stage j complete; later ones may fly
      const int later = min(nk - 1, j + STAGES - 3) - j;
      switch (later) {  // vmcnt needs an immediate
        case 0: wait_vm_barrier<0>(); break;
        case 1: wait_vm_barrier<DPW>(); break;
        case 2: wait_vm_barrier<2 * DPW>(); break;
        case 3: wait_vm_barrier<3 * DPW>(); break;
        default: wait_vm_barrier<4 * DPW>(); break;
      }
    };
#pragma unroll
    for (int i = 0; i < STAGES; ++i)
      if (i < nk) issue(i);
    // stages 0 and 1 visible
    {
      const int later = min(nk - 1, STAGES - 1) - 1;  // issued after stage 1
      if (later <= 0) wait_vm_barrier<0>();
      else if (later == 1) wait_vm_barrier<DPW>();
      else if (later == 2) wait_vm_barrier<2 * DPW>();
      else wait_vm_barrier<3 * DPW>();
    }
    Frags F0, F1;
    if (JN > 0) load_frags(0, F0);
    auto step = [&](int kt, Frags& cur, Frags& nxt) {
      if (JN > 0) {
        // the last step re-reads the final stage (valid, no longer refilled)
        load_frags(min(kt + 1, nk - 1), nxt);
        mfma_stage(cur);
      }
      if (kt + 2 < nk)
        wait_for(kt + 2);
      else
        wait_vm_barrier<0>();
      if (kt + STAGES < nk) issue(kt + STAGES);
    };
    // nk is even (K is a multiple of 64), so the two-step body needs no guard
    for (int kt = 0; kt < nk; kt += 2) {
      step(kt, F0, F1);
      step(kt + 1, F1, F0);
    }
  };
  switch (jn) {
    case 0: main_loop(std::integral_constant<int, 0>()); break;
    case 1: main_loop(std::integral_constant<int, 1>()); break;
    case 2: main_loop(std::integral_constant<int, (WB >= 2 ? 2 : 1)>()); break;
    case 3: main_loop(std::integral_constant<int, (WB >= 3 ? 3 : 1)>()); break;
    default: main_loop(std::integral_constant<int, WB>()); break;
  }

  // ---- epilogue: acc[i][j][4 g + r] = C[fragment-i row 8 g + 4 (lane >> 5) + r]
  // [token fragment j, token lane & 31]: four consecutive output features per
  // group g, stored as one 8-byte vector.
#pragma unroll
  for (int j = 0; j < WB; ++j) {
    const int row = row0 + tok0 + 32 * j + (lane & 31);
    if (j >= jn || row >= row_end) continue;
    uint16_t* orow = out + (size_t)row * N;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (GATED) {
#pragma unroll
        for (int i = 0; i < WA / 2; ++i) {
          const int n = n0 + wn * 16 * WA + 32 * i + 8 * g + 4 * lk;
          if (n >= N) continue;
          float hv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float gt = acc[i][j][4 * g + r], up = acc[i + WA / 2][j][4 * g + r];
            hv[r] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
          }
          u32x2 pk;
          pk.x = pack_bf16x2(hv[0], hv[1]);
          pk.y = pack_bf16x2(hv[2], hv[3]);
          *reinterpret_cast<u32x2*>(orow + n) = pk;
        }
      } else {
#pragma unroll
        for (int i = 0; i < WA; ++i) {
          const int n = n0 + wn * 32 * WA + 32 * i + 8 * g + 4 * lk;
          if (n >= N) continue;
          u32x2 pk;
          pk.x = pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
          pk.y = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
          *reinterpret_cast<u32x2*>(orow + n) = pk;
        }
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
// Tile choice.  256x256 tiles (128x128 per wave) halve LDS fragment traffic
// per flop; they are used unless they would leave fewer than ~2 blocks per CU,
// in which case 256 weight rows x 128 tokens keep the grid full.
struct GemmPlan {
  int wb;       // token fragments per wave (4: 256-token tiles, 2: 128-token tiles)
  int n_tiles;  // weight tiles over N
  int blocks;   // grid size (multiple of 8, worst case over any row table)
};

static GemmPlan plan_gemm(long rows, int E, int N, bool gated) {
  const int tn = gated ? 128 : 256;
  GemmPlan p;
  p.n_tiles = div_up(N, tn);
  const int cus = 256;
  const long avg = (rows + E - 1) / E;  // typical rows per expert
  const long est256 = (long)p.n_tiles * E * ((avg + 255) / 256);
  // many rows per expert: MFMA-bound, big tiles; otherwise weight streaming
  p.wb = (avg >= 512 && est256 >= 2 * cus) ? 4 : 2;
  (void)cus;
  const long total = (long)p.n_tiles * worst_row_tiles(rows, E, 64 * p.wb);
  p.blocks = (int)((total + 7) / 8 * 8);
  return p;
}

template <bool GATED>
static void launch_gemm(const GemmPlan& p, const uint16_t* act, const int32_t* offs,
                        const uint16_t* w0, const uint16_t* w1, uint16_t* out, int E, int N, int K,
                        int rows, hipStream_t st) {
  const int band = 8;
  if (p.wb == 4)
    grouped_gemm_bf16_kernel<GATED, 4, 4><<<p.blocks, 256, 0, st>>>(
        act, offs, w0, w1, out, E, N, K, rows, p.n_tiles, band);
  else
    grouped_gemm_bf16_kernel<GATED, 4, 2><<<p.blocks, 256, 0, st>>>(
        act, offs, w0, w1, out, E, N, K, rows, p.n_tiles, band);
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
  const GemmPlan p = plan_gemm(rows, c.E, c.f, true);
  launch_gemm<true>(p, static_cast<const uint16_t*>(x_perm), offs,
                    static_cast<const uint16_t*>(wg), static_cast<const uint16_t*>(wu),
                    static_cast<uint16_t*>(h), c.E, c.f, c.d, (int)rows, st);
  return hipGetLastError();
}

// out[rows, N] = act[rows, K] W_e^T by expert row segments, W_e [N, K] (bf16).
hipError_t launch_grouped_linear(const moe_config& c, const uint16_t* act, const int32_t* offs,
                                 const uint16_t* w, uint16_t* out, int N, int K, hipStream_t st) {
  const long rows = (long)c.T * c.k;
  const GemmPlan p = plan_gemm(rows, c.E, N, false);
  launch_gemm<false>(p, act, offs, w, nullptr, out, c.E, N, K, (int)rows, st);
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
  const GemmPlan p = plan_gemm(rows, c.E, c.d, false);
  launch_gemm<false>(p, static_cast<const uint16_t*>(h), offs, static_cast<const uint16_t*>(wd),
                     nullptr, static_cast<uint16_t*>(y), c.E, c.d, c.f, (int)rows, st);
  return hipGetLastError();
}

}  // namespace moe
