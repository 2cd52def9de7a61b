// Layer backward on the cached routing.
//
// Pages: [SyncTax] §2.4 (the backward retraces the forward's routing from the
// routing indices kept by the forward; it is the forward's mirror) and
// [V4-overlap], PP bubble section (a layer's backward turns dy into dx and the
// weight gradient dW = x^T dy).  Every product C = A B of the forward gives
// dA = dC B^T and dB = A^T dC:
//   combine    out[t] = sum_j g[t,j] y[p(t,j)]:
//              dy[p(t,j)] = g[t,j] dout[t],  dg[t,j] = <dout[t], y[p(t,j)]>
//   down       y = h Wd^T:       dh = dy Wd,   dWd_e = dy_e^T h_e
//   SwiGLU     h = SiLU(a) u:    da = dh u SiLU'(a),  du = dh SiLU(a),
//              SiLU'(a) = sig(a) (1 + a (1 - sig(a)))
//   gate/up    a = x Wg^T, u = x Wu^T:  dx = da Wg + du Wu,
//              dWg_e = da_e^T x_e,  dWu_e = du_e^T x_e
//   dispatch   x_perm[p] = x[src(p)]:  dx[t] = sum of the k rows of token t
//   gates      softmax of s = z + b over the support set S (the k chosen, the
//              P pre-selected, or all E): ds_l = q_l (dq_l - sum_j g_j dg_j)
//              on S; dz = ds, db = sum_t dz[t];  z = x Wr^T: dx += dz Wr,
//              dWr = dz^T x.
//
// gfx950 design
//  * Two MFMA kernels serve every backward product.  dgrad (dh, dx, the
//    router's dz Wr) runs over the expert row segments with the forward's
//    device tile table; wgrad (dW) runs per expert with the expert's row
//    segment as the reduction (zeros for an expert without rows).
//  * Both stream their operands into LDS with the gfx950 LDS-DMA load (no
//    staging registers) through a ring of four 32-k stages with explicit
//    waits.  Operands whose k is contiguous (dgrad's activation rows) sit in
//    LDS as 64-byte rows and are read as 16-byte fragments; operands whose k
//    is the slow index (dgrad's weights, both wgrad operands) are copied as
//    they lie and read transposed with ds_read_b64_tr_b16.
//  * 128 x 128 tiles (four waves of 64 x 64, two blocks per CU); the wgrad
//    also has 256 x 256 (eight waves, one block per CU, half the L2 traffic)
//    for long reductions.
//  * Rows and columns past a tile's end are clamped onto data inside the
//    buffers (they only feed outputs that are never stored); k past the end
//    of a part or an expert's segment is read from a page of zeros.
#include <cmath>
#include <type_traits>

#include "common.h"
#include "tiles.h"

namespace moe {

struct GemmPart {
  const uint16_t* a;
  const uint16_t* b;
  long lda, ldb;   // leading dimensions in elements
  long b_estride;  // elements between two experts' weight matrices
  int K;           // k extent of this part
};

struct GemmArgs {  // dgrad
  GemmPart part[2];
  int nparts;
  uint16_t* c;
  long ldc;
  const int32_t* offs;
  int E, rows;
  int N;
  int n_tiles, band;
};

// ---------------------------------------------------------------- wgrad, LDS-DMA
// C_e[M, N] = sum over the expert's rows r of A[r, m] B[r, n].  Both operands
// have k (the row index) as their slow index, so they go to LDS as they are
// laid out in memory -- by the gfx950 LDS-DMA load, no staging registers --
// and the MFMA fragments are read transposed with ds_read_b64_tr_b16: within
// each 16-lane group, lane c receives element c % 4 of the 8-byte pieces
// addressed by lanes 4 q + c / 4 (q = 0..3), so when lane 4 q + j addresses
// k-row k0 + q, columns c0 + 4 j .. + 3, lane c gets column c0 + c at the four
// k-rows k0 .. k0 + 3.  Two such reads give an MFMA lane its 8 consecutive k.
// 128 x 128 tiles, four waves of 64 x 64, 32-row k stages in a ring of four
// (64 KB, two blocks per CU), explicit waits.  k-rows past the expert's end are
// copied from a page of zeros; columns past M or N are clamped inside the
// row (they only feed outputs that are never stored).
typedef __attribute__((address_space(3))) void bw_lds_t;
typedef short bw_v4i16 __attribute__((ext_vector_type(4)));

__device__ __attribute__((aligned(16))) const uint32_t kBwZeroPage[4] = {0u, 0u, 0u, 0u};

__device__ __forceinline__ uint32_t bw_lds_addr(const void* p) {
  return (uint32_t)(size_t)(const bw_lds_t*)p;
}
// 16 bytes per lane, global -> LDS; lane L writes LDS bytes [lds + 16 L, + 16).
__device__ __forceinline__ void bw_dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void bw_wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

constexpr int kWK = 32;                      // k-rows per stage
constexpr int kWRing = 4;                    // stages in the LDS ring
constexpr int kWDpw = 4;                     // DMA instructions (1 KB) per wave per stage

// byte offset of 16-byte column piece p of k-row r in one operand's stage
// (2 WT bytes per k-row; pieces XOR-swizzled with (r & 3) << 2 so that a
// transposed read's four k-rows land on different banks)
template <int WT>
__device__ __forceinline__ uint32_t wg_piece(int r, int p) {
  return (uint32_t)(r * (2 * WT) + ((p ^ ((r & 3) << 2)) << 4));
}

// <TM, TN>: tile of TM rows of C (A columns) by TN columns (B columns).
// 128 x 128: four waves of 64 x 64, 64 KB ring, two blocks per CU, the next
// stage's fragments read while the current one's MFMAs run.  256 x 256: eight
// waves of 128 x 64, 128 KB ring, one block per CU, half the operand bytes
// per flop.  256 x 128: four waves of 128 x 64, a ring of three (72 KB), two
// blocks per CU, a quarter fewer operand bytes per flop.  The larger wave
// tiles keep one fragment set (two would not fit their registers).
// F32OUT: C is float32 (the partial sums of a reduction split over row
// segments), else bf16.
template <int TM, int TN, bool F32OUT = false>
__global__ __launch_bounds__(TN == 256 ? 512 : 256, TN == 256 ? 1 : 2) void wgrad_dma_kernel(
    const uint16_t* __restrict__ a, long lda, const uint16_t* __restrict__ b, long ldb,
    const int32_t* __restrict__ offs, int E, int rows, int M, int N, int m_tiles, int n_tiles,
    void* __restrict__ c, long ldc, long c_estride) {
  constexpr int NW = TN == 256 ? 8 : 4;        // waves
  constexpr int WN = NW / 2;                   // waves along N; two along M
  constexpr int FM = TM / 64;                  // 32-column A fragments per wave
  constexpr int RING = TM == 256 && TN == 128 ? 3 : kWRing;
  constexpr int OPA = kWK * TM * 2;            // A's stage
  constexpr int OPB = kWK * TN * 2;            // B's stage
  constexpr int STB = OPA + OPB;               // one stage
  constexpr int CA = OPA / 1024;               // 1 KB chunks of A
  constexpr int RPCA = 1024 / (2 * TM), RPCB = 1024 / (2 * TN);  // k-rows per chunk
  constexpr int DPW = (STB / 1024) / NW;       // DMA instructions per wave per stage
  constexpr bool kPrefetch = TM == 128;
  static_assert((STB / 1024) % NW == 0, "chunks per stage");
  static_assert(WN * 64 == TN, "wave columns");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[RING * STB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int per_e = m_tiles * n_tiles;
  const int e = blockIdx.x / per_e;
  const int rr = blockIdx.x - e * per_e;
  const int m0 = (rr / n_tiles) * TM, n0 = (rr % n_tiles) * TN;
  const int m_lim = min(TM, M - m0), n_lim = min(TN, N - n0);
  const int k0 = min(max(offs[e], 0), rows);
  const int k_lim = min(max(offs[e + 1], k0), rows) - k0;
  const int nk = (k_lim + kWK - 1) / kWK;

  // ---- DMA: stage chunk q (1 KB): A chunks first (RPCA k-rows each), then B
  // (RPCB each); wave w issues chunks w + NW i.  Lane L lands at k-row
  // RPC (chunk) + L / (width / 8), physical piece L % (width / 8), so it
  // fetches logical piece (L % (width / 8)) ^ ((row & 3) << 2).
  int drow[DPW];
  const uint16_t* dcol[DPW];
  long dld[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int q = wave + NW * i;
    const bool is_a = q < CA;
    const int width = is_a ? TM : TN;
    const int r = is_a ? RPCA * q + lane / (TM / 8) : RPCB * (q - CA) + lane / (TN / 8);
    const int p = (lane % (width / 8)) ^ ((r & 3) << 2);
    const int lim = is_a ? m_lim : n_lim;  // a multiple of 8
    const int col = min(8 * p, lim - 8);
    drow[i] = r;
    dcol[i] = is_a ? a + (size_t)k0 * lda + m0 + col : b + (size_t)k0 * ldb + n0 + col;
    dld[i] = is_a ? lda : ldb;
  }
  const uint32_t lds0 = bw_lds_addr(ring);
  auto issue = [&](int kt) {
    const uint32_t sbase = lds0 + (uint32_t)(kt % RING) * STB;
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int k = kt * kWK + drow[i];
      const void* src = k < k_lim ? (const void*)(dcol[i] + (size_t)k * dld[i])
                                  : (const void*)kBwZeroPage;
      bw_dma16(src, sbase + (uint32_t)(wave + NW * i) * 1024u);
    }
  };

  // ---- fragments: wave (wm, wn) owns A columns wm*TM/2.. and B columns wn*64..
  const int wm = wave / WN, wn = wave % WN;
  const int g = lane >> 4;
  const int tr_col = 16 * (g & 1) + 4 * (lane & 3);  // column of the addressed piece
  const int tr_row = 8 * (g >> 1) + ((lane >> 2) & 3);
  struct Frags {
    bf16x8 a[2][FM];  // [k slab][fragment]
    bf16x8 b[2][2];
  };
  auto read_frag = [&](uint32_t opbase, int col0, int s2, auto width_c) -> bf16x8 {
    constexpr int W = decltype(width_c)::value;
    const int col = col0 + tr_col;
    bw_v4i16 h[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int r = 16 * s2 + tr_row + 4 * hh;
      const uint32_t addr = opbase + wg_piece<W>(r, col >> 3) + (uint32_t)((col & 7) * 2);
      h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) bw_v4i16*)(size_t)addr);
    }
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
    return __builtin_bit_cast(bf16x8, v);
  };
  auto load_frags = [&](int kt, Frags& F) {
    const uint32_t sb = lds0 + (uint32_t)(kt % RING) * STB;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        F.a[s2][i] = read_frag(sb, wm * (TM / 2) + 32 * i, s2, std::integral_constant<int, TM>());
#pragma unroll
      for (int j = 0; j < 2; ++j)
        F.b[s2][j] = read_frag(sb + OPA, wn * 64 + 32 * j, s2, std::integral_constant<int, TN>());
    }
  };
  f32x16 acc[FM][2];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  auto mfma_stage = [&](const Frags& F) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.b[s2][j], F.a[s2][i], acc[i][j],
                                                              0, 0, 0);
  };
  // Stage j lives in ring slot j % RING.  With prefetch, stage kt's fragments are
  // read during step kt - 1; without, at the start of step kt.  End of step
  // kt: wait for this wave's copies of stage kt + 2 (kt + 1 without
  // prefetch), barrier (that stage visible; slot kt % 4 no longer read),
  // refill slot kt % 4 with stage kt + 4.
  constexpr int AHEAD = kPrefetch ? 2 : 1;
  if (nk > 0) {
#pragma unroll
    for (int i = 0; i < RING; ++i)
      if (i < nk) issue(i);
    {  // stages 0 .. AHEAD - 1 visible, the later ones may still fly
      const int later = min(nk - 1, RING - 1) - (AHEAD - 1);
      if (later <= 0) bw_wait_vm_barrier<0>();
      else if (later == 1) bw_wait_vm_barrier<DPW>();
      else if (later == 2) bw_wait_vm_barrier<2 * DPW>();
      else bw_wait_vm_barrier<3 * DPW>();
    }
    auto finish = [&](int kt) {
      const int j = kt + AHEAD;  // the stage that must be visible next
      const int later = j < nk ? min(nk - 1, kt + RING - 1) - j : 0;
      if (later <= 0) bw_wait_vm_barrier<0>();
      else if (later == 1) bw_wait_vm_barrier<DPW>();
      else bw_wait_vm_barrier<2 * DPW>();
      if (kt + RING < nk) issue(kt + RING);
    };
    if constexpr (kPrefetch) {
      Frags F0, F1;
      load_frags(0, F0);
      auto step = [&](int kt, Frags& cur, Frags& nxt) {
        load_frags(min(kt + 1, nk - 1), nxt);  // the last step re-reads the final stage
        mfma_stage(cur);
        finish(kt);
      };
      for (int kt = 0; kt < nk; kt += 2) {
        step(kt, F0, F1);
        if (kt + 1 < nk) step(kt + 1, F1, F0);
      }
    } else {
      for (int kt = 0; kt < nk; ++kt) {
        Frags F;
        load_frags(kt, F);
        mfma_stage(F);
        finish(kt);
      }
    }
  }

  // ---- epilogue: acc[i][j][4 gq + r] = C[m = wm*TM/2 + 32 i + (lane & 31)]
  // [n = wn*64 + 32 j + 8 gq + 4 (lane >> 5) + r]
  const int lk = lane >> 5;
  if constexpr (!F32OUT) {
    // Staged through the (drained) ring: rows of TN bf16 padded to a 16-byte
    // multiple, then every lane stores one 16-byte piece, TN / 8 lanes per
    // row, so a wave writes whole rows instead of 16 bytes in each of 32
    // rows.  A tile that does not fit the ring goes in two halves of rows
    // (the waves with wm = 0, then those with wm = 1).
    constexpr int PITCH = TN * 2 + 16;
    constexpr int PPR = TN / 8;  // 16-byte pieces per row
    constexpr int HALVES = TM * PITCH <= RING * STB ? 1 : 2;
    constexpr int RH = TM / HALVES;  // rows per pass
    static_assert(RH * PITCH <= RING * STB, "the staged rows fit the ring");
    uint16_t* cb = static_cast<uint16_t*>(c) + (size_t)e * c_estride + (size_t)m0 * ldc + n0;
    const int p = tid % PPR;
    __syncthreads();  // every wave is done reading the ring
#pragma unroll
    for (int hv = 0; hv < HALVES; ++hv) {
      if (HALVES == 1 || wm == hv) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int m = wm * (TM / 2) + 32 * i + (lane & 31) - hv * RH;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int n = wn * 64 + 32 * j + 8 * gq + 4 * lk;
              u32x2 pk;
              pk.x = pack_bf16x2(acc[i][j][4 * gq], acc[i][j][4 * gq + 1]);
              pk.y = pack_bf16x2(acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]);
              *reinterpret_cast<u32x2*>(ring + m * PITCH + n * 2) = pk;
            }
        }
      }
      __syncthreads();
#pragma unroll 4
      for (int r = tid / PPR; r < RH; r += NW * 64 / PPR)
        if (hv * RH + r < m_lim && 8 * p < n_lim)
          *reinterpret_cast<u32x4*>(cb + (size_t)(hv * RH + r) * ldc + 8 * p) =
              *reinterpret_cast<const u32x4*>(ring + r * PITCH + 16 * p);
      if (hv + 1 < HALVES) __syncthreads();  // the next half overwrites these rows
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = wm * (TM / 2) + 32 * i + (lane & 31);
    if (m >= m_lim) continue;
    const size_t crow = (size_t)e * c_estride + (size_t)(m0 + m) * ldc + n0;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int n = wn * 64 + 32 * j + 8 * gq + 4 * lk;
        if (n >= n_lim) continue;
        if constexpr (F32OUT) {
          float4 v;
          v.x = acc[i][j][4 * gq];
          v.y = acc[i][j][4 * gq + 1];
          v.z = acc[i][j][4 * gq + 2];
          v.w = acc[i][j][4 * gq + 3];
          *reinterpret_cast<float4*>(static_cast<float*>(c) + crow + n) = v;
        } else {
          u32x2 pk;
          pk.x = pack_bf16x2(acc[i][j][4 * gq], acc[i][j][4 * gq + 1]);
          pk.y = pack_bf16x2(acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]);
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(c) + crow + n) = pk;
        }
      }
  }
}

// ---------------------------------------------------------------- dgrad, LDS-DMA
// C[rows, N] = A[rows, K] B_e[K, N] (+ a second part with the same leading
// dimensions) over the expert row segments.  A (k contiguous) is copied to LDS
// in 64-byte rows of 32 k (16-byte pieces XOR-swizzled with (row >> 2) & 3)
// and read as 16-byte fragments; B (the expert's weights, n contiguous) is
// copied as it lies and read transposed (ds_read_b64_tr_b16), as in the
// wgrad.  128 x 128 tiles placed by the device tile table, four waves of
// 64 x 64, 32-k stages in a ring of four, explicit waits, rows past the
// tile's end clamped onto its last row, k past a part's end read from the
// zero page.
__global__ __launch_bounds__(256, 2) void dgrad_dma_kernel(GemmArgs g) {
  constexpr int WT = 128;
  constexpr int OPB = kWK * WT * 2;  // one operand's stage: 8 KB
  constexpr int STB = 2 * OPB;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kWRing * STB];
  __shared__ int s_tile[4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wave == 0) place_tile<WT>(g.offs, g.E, g.rows, g.n_tiles, g.band, lane, s_tile);
  __syncthreads();
  const int e = s_tile[0];
  if (e < 0) return;  // block-uniform
  const int m0 = s_tile[1], m_lim = s_tile[2] - s_tile[1], n0 = s_tile[3] * WT;
  const int n_lim = min(WT, g.N - n0);
  const int K0 = g.part[0].K, K1 = g.nparts > 1 ? g.part[1].K : 0;
  const int nst0 = (K0 + kWK - 1) / kWK;
  const int nk = nst0 + (K1 + kWK - 1) / kWK;
  const long lda = g.part[0].lda, ldb = g.part[0].ldb, bes = g.part[0].b_estride;

  // ---- DMA: chunks 0..7 = A (16 rows of 64 bytes each), 8..15 = B (4 k-rows
  // of 256 bytes each); wave w issues chunks w + 4 i.
  uint32_t doff[kWDpw];  // element offset of this lane's piece inside the part's stage
  int dk[kWDpw];         // k of this lane's piece inside the stage
#pragma unroll
  for (int i = 0; i < kWDpw; ++i) {
    const int q = wave + 4 * i;
    if (q < 8) {  // A: row 16 q + L / 4, physical piece L % 4
      const int r = 16 * q + (lane >> 2);
      const int lp = (lane & 3) ^ ((lane >> 4) & 3);
      dk[i] = 8 * lp;
      doff[i] = (uint32_t)((long)min(r, m_lim - 1) * lda + 8 * lp);
    } else {  // B: k-row 4 (q - 8) + L / 16, physical piece L % 16
      const int r = 4 * (q - 8) + (lane >> 4);
      const int p = (lane & 15) ^ ((r & 3) << 2);
      dk[i] = r;
      doff[i] = (uint32_t)((long)r * ldb + min(8 * p, n_lim - 8));
    }
  }
  const uint32_t lds0 = bw_lds_addr(ring);
  auto issue = [&](int kt) {
    const bool p1 = kt >= nst0;
    const int ks = (kt - (p1 ? nst0 : 0)) * kWK;
    const int klim = p1 ? K1 : K0;
    const uint16_t* abase = (p1 ? g.part[1].a : g.part[0].a) + (size_t)m0 * lda + ks;
    const uint16_t* bbase = (p1 ? g.part[1].b : g.part[0].b) + (size_t)e * bes + n0 +
                            (size_t)ks * ldb;
    const uint32_t sbase = lds0 + (uint32_t)(kt % kWRing) * STB;
#pragma unroll
    for (int i = 0; i < kWDpw; ++i) {
      const int q = wave + 4 * i;
      const uint16_t* base = q < 8 ? abase : bbase;
      const void* src = ks + dk[i] < klim ? (const void*)(base + doff[i])
                                          : (const void*)kBwZeroPage;
      bw_dma16(src, sbase + (uint32_t)q * 1024u);
    }
  };

  // ---- fragments
  const int wm = wave >> 1, wn = wave & 1;
  const int lk = lane >> 5;
  const int gq4 = lane >> 4;
  const int tr_col = 16 * (gq4 & 1) + 4 * (lane & 3);
  const int tr_row = 8 * (gq4 >> 1) + ((lane >> 2) & 3);
  struct Frags {
    bf16x8 a[2][2];
    bf16x8 b[2][2];
  };
  auto load_frags = [&](int kt, Frags& F) {
    const uint32_t sb = lds0 + (uint32_t)(kt % kWRing) * STB;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int qa = 2 * s2 + lk;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + 32 * i + (lane & 31);
        const uint32_t off = (sb - lds0) + (uint32_t)((r * 4 + (qa ^ ((r >> 2) & 3))) * 16);
        F.a[s2][i] = *reinterpret_cast<const bf16x8*>(ring + off);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = wn * 64 + 32 * j + tr_col;
        bw_v4i16 h[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int r = 16 * s2 + tr_row + 4 * hh;
          const uint32_t addr = sb + OPB + wg_piece<WT>(r, col >> 3) + (uint32_t)((col & 7) * 2);
          h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) bw_v4i16*)(size_t)addr);
        }
        typedef short v8i16 __attribute__((ext_vector_type(8)));
        const v8i16 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
        F.b[s2][j] = __builtin_bit_cast(bf16x8, v);
      }
    }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  auto mfma_stage = [&](const Frags& F) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.b[s2][j], F.a[s2][i], acc[i][j],
                                                              0, 0, 0);
  };
  // same ring discipline as the wgrad with prefetch: stage kt's fragments are
  // read during step kt - 1; the end of step kt makes stage kt + 2 visible and
  // refills slot kt % 4 with stage kt + 4
  if (nk > 0) {
#pragma unroll
    for (int i = 0; i < kWRing; ++i)
      if (i < nk) issue(i);
    {
      const int later = min(nk - 1, kWRing - 1) - 1;
      if (later <= 0) bw_wait_vm_barrier<0>();
      else if (later == 1) bw_wait_vm_barrier<kWDpw>();
      else bw_wait_vm_barrier<2 * kWDpw>();
    }
    auto finish = [&](int kt) {
      const int j = kt + 2;
      const int later = j < nk ? min(nk - 1, kt + kWRing - 1) - j : 0;
      if (later <= 0) bw_wait_vm_barrier<0>();
      else bw_wait_vm_barrier<kWDpw>();
      if (kt + kWRing < nk) issue(kt + kWRing);
    };
    Frags F0, F1;
    load_frags(0, F0);
    auto step = [&](int kt, Frags& cur, Frags& nxt) {
      load_frags(min(kt + 1, nk - 1), nxt);
      mfma_stage(cur);
      finish(kt);
    };
    for (int kt = 0; kt < nk; kt += 2) {
      step(kt, F0, F1);
      if (kt + 1 < nk) step(kt + 1, F1, F0);
    }
  }

  // ---- epilogue: C[row m0 + m][n0 + n], staged through the drained ring
  // like the wgrad's (rows padded to 272 bytes), then 16 lanes per row store
  // it in 16-byte pieces.
  constexpr int PITCH = WT * 2 + 16;
  static_assert(WT * PITCH <= kWRing * STB, "the staged tile fits the ring");
  __syncthreads();  // every wave is done reading the ring
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = wm * 64 + 32 * i + (lane & 31);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int n = wn * 64 + 32 * j + 8 * gq + 4 * lk;
        u32x2 pk;
        pk.x = pack_bf16x2(acc[i][j][4 * gq], acc[i][j][4 * gq + 1]);
        pk.y = pack_bf16x2(acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]);
        *reinterpret_cast<u32x2*>(ring + m * PITCH + n * 2) = pk;
      }
  }
  __syncthreads();
  uint16_t* cb = g.c + (size_t)m0 * g.ldc + n0;
  const int p = tid % (WT / 8);
#pragma unroll 4
  for (int r = tid / (WT / 8); r < WT; r += 256 / (WT / 8))
    if (r < m_lim && 8 * p < n_lim)
      *reinterpret_cast<u32x4*>(cb + (size_t)r * g.ldc + 8 * p) =
          *reinterpret_cast<const u32x4*>(ring + r * PITCH + 16 * p);
}

// dgrad: C[rows, N] = A[rows, K] B_e[K, N] (+ the second part), by expert
// row segments.  Every K, N and leading dimension is a multiple of 8.
// wgrad: 256-wide tiles when they still give every CU a tile, else 128-wide.
constexpr int kCUs = 256;

static hipError_t launch_dgrad(const GemmPart* parts, int nparts, const int32_t* offs, int E,
                               int rows, int N, uint16_t* c, long ldc, hipStream_t st) {
  if (nparts == 2 && (parts[1].lda != parts[0].lda || parts[1].ldb != parts[0].ldb ||
                      parts[1].b_estride != parts[0].b_estride))
    return hipErrorInvalidValue;  // the kernel reads these from the first part
  GemmArgs g{};
  for (int p = 0; p < nparts; ++p) g.part[p] = parts[p];
  g.nparts = nparts;
  g.c = c;
  g.ldc = ldc;
  g.offs = offs;
  g.E = E;
  g.rows = rows;
  g.N = N;
  g.band = 8;
  // 128-wide tiles: the 256-wide dgrad tile measured no faster (and does not
  // fit its registers without spilling)
  g.n_tiles = div_up(N, 128);
  const long total = (long)g.n_tiles * worst_row_tiles(rows, E, 128);
  dgrad_dma_kernel<<<(int)((total + 7) / 8 * 8), 256, 0, st>>>(g);
  return hipGetLastError();
}

// wgrad: C_e[M, N] = A_rows^T B_rows over expert e's row segment, for every
// expert (zeros for an expert without rows).
static hipError_t launch_wgrad(const uint16_t* a, long lda, const uint16_t* b, long ldb,
                               const int32_t* offs, int E, int rows, int M, int N, uint16_t* c,
                               long ldc, long c_estride, hipStream_t st) {
  // Long reductions (from ~1024 rows per expert): 256 x 256 where such tiles
  // fill the chip; short ones: 256 x 128 (two blocks per CU) where those
  // fill it twice over; else 128 x 128.
  const long t256 = (long)E * div_up(M, 256) * div_up(N, 256);
  const long t256x128 = (long)E * div_up(M, 256) * div_up(N, 128);
  if (rows >= 1024L * E && t256 >= kCUs) {
    const int mt = div_up(M, 256), nt = div_up(N, 256);
    wgrad_dma_kernel<256, 256><<<(int)t256, 512, 0, st>>>(a, lda, b, ldb, offs, E, rows, M, N,
                                                          mt, nt, c, ldc, c_estride);
  } else if (t256x128 >= 2L * kCUs) {
    const int mt = div_up(M, 256), nt = div_up(N, 128);
    wgrad_dma_kernel<256, 128><<<(int)t256x128, 256, 0, st>>>(a, lda, b, ldb, offs, E, rows, M,
                                                              N, mt, nt, c, ldc, c_estride);
  } else {
    const int mt = div_up(M, 128), nt = div_up(N, 128);
    wgrad_dma_kernel<128, 128><<<(int)((long)E * mt * nt), 256, 0, st>>>(
        a, lda, b, ldb, offs, E, rows, M, N, mt, nt, c, ldc, c_estride);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------- combine backward
// One wave per token: dy[p(t,j)] = bf16(g dout[t]); dg[t,j] = <dout[t], y[p(t,j)]>
// (fp32, lane partials then a fixed xor tree).
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// One wave per token.  VR > 0 (rows of up to 64 VR vectors): the token's
// d_out row stays in registers and each chosen row's vectors are all loaded
// before they are used; VR = 0: one vector at a time.  Either way a lane
// accumulates its dot product over the same vectors in the same order.
template <int VR>
__global__ __launch_bounds__(256) void combine_backward_kernel(
    const u32x4* __restrict__ dout, const u32x4* __restrict__ y, const int32_t* __restrict__ slot_of,
    const float* __restrict__ topk_w, u32x4* __restrict__ dy, float* __restrict__ dg, int T, int k,
    int nvec, int A) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave
  const u32x4* drow = dout + (size_t)t * nvec;
  auto body = [&](const u32x4& a, const u32x4& b, float w, float& dot) {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a0 = bf16_lo(a[q]), a1 = bf16_hi(a[q]);
      dot = fmaf(a0, bf16_lo(b[q]), dot);
      dot = fmaf(a1, bf16_hi(b[q]), dot);
      o[q] = pack_bf16x2(w * a0, w * a1);
    }
    return o;
  };
  if constexpr (VR > 0) {
    u32x4 a[VR];
#pragma unroll
    for (int i = 0; i < VR; ++i)
      if (lane + 64 * i < nvec) a[i] = drow[lane + 64 * i];
    for (int j = 0; j < k; ++j) {
      const int p = min(max(slot_of[(size_t)t * k + j], 0), A - 1);
      const float w = topk_w[(size_t)t * k + j];
      const u32x4* yrow = y + (size_t)p * nvec;
      u32x4* dyrow = dy + (size_t)p * nvec;
      u32x4 b[VR];
#pragma unroll
      for (int i = 0; i < VR; ++i)
        if (lane + 64 * i < nvec) b[i] = yrow[lane + 64 * i];
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < VR; ++i)
        if (lane + 64 * i < nvec) dyrow[lane + 64 * i] = body(a[i], b[i], w, dot);
      dot = wave_sum_f(dot);
      if (lane == 0) dg[(size_t)t * k + j] = dot;
    }
  } else {
    for (int j = 0; j < k; ++j) {
      const int p = min(max(slot_of[(size_t)t * k + j], 0), A - 1);
      const float w = topk_w[(size_t)t * k + j];
      const u32x4* yrow = y + (size_t)p * nvec;
      u32x4* dyrow = dy + (size_t)p * nvec;
      float dot = 0.f;
      for (int v = lane; v < nvec; v += 64) dyrow[v] = body(drow[v], yrow[v], w, dot);
      dot = wave_sum_f(dot);
      if (lane == 0) dg[(size_t)t * k + j] = dot;
    }
  }
}

// ------------------------------------------------------------- SwiGLU backward
// Per element: h = SiLU(a) u; da = dh u SiLU'(a); du = dh SiLU(a).
// dh and h share one buffer (element i read, then written, by one thread);
// da and du go side by side into one [rows, 2 f] buffer (row r: da_r, du_r),
// the activation operand of dx = [da du] [W_g; W_u].  fv = f / 8.
__global__ __launch_bounds__(256) void swiglu_backward_kernel(const u32x4* a_in, const u32x4* u_in,
                                                              u32x4* dh_h,
                                                              u32x4* __restrict__ dadu, long fv,
                                                              long nvec) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= nvec) return;
  const u32x4 va = a_in[i], vu = u_in[i], vd = dh_h[i];
  u32x4 oh, oa, ou;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float r[2][3];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const float a = hh ? bf16_hi(va[q]) : bf16_lo(va[q]);
      const float u = hh ? bf16_hi(vu[q]) : bf16_lo(vu[q]);
      const float d = hh ? bf16_hi(vd[q]) : bf16_lo(vd[q]);
      const float sig = 1.0f / (1.0f + expf(-a));
      const float silu = a * sig;
      r[hh][0] = silu * u;
      r[hh][1] = d * u * sig * (1.0f + a * (1.0f - sig));
      r[hh][2] = d * silu;
    }
    oh[q] = pack_bf16x2(r[0][0], r[1][0]);
    oa[q] = pack_bf16x2(r[0][1], r[1][1]);
    ou[q] = pack_bf16x2(r[0][2], r[1][2]);
  }
  const long r = i / fv, cv = i - r * fv;
  dh_h[i] = oh;
  dadu[r * 2 * fv + cv] = oa;
  dadu[r * 2 * fv + fv + cv] = ou;
}

// ------------------------------------------------------------- gates backward
// One wave per token, EPL experts per lane.  q = softmax of s = z + b over the
// support set, m = s of the first chosen expert; dq_e = dg_j for the j-th
// chosen expert; ds_e = q_e (dq_e - sum_e' q_e' dq_e') on the support, 0
// elsewhere.  The pre-selected set (presel > 0, no renormalisation) is the
// top presel experts by (s desc, e asc), ranked in LDS.
template <int EPL>
__global__ __launch_bounds__(256) void gates_backward_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ dg, int T, int E, int k,
    int presel, int renorm, float* __restrict__ dz, uint16_t* __restrict__ dz_bf16) {
  extern __shared__ float s_sc[];  // [4 waves][E], for the pre-selection ranks
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + w;
  const bool live = t < T;  // wave-uniform
  const bool rank_sel = !renorm && presel > 0;
  float sc[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    sc[i] = -INFINITY;
    if (live && e < E) {
      const float z = logits[(size_t)t * E + e];
      sc[i] = bias ? z + bias[e] : z;
      if (rank_sel) s_sc[w * E + e] = sc[i];
    }
  }
  __syncthreads();
  if (!live) return;
  const int* idx = topk_idx + (size_t)t * k;
  const int first = min(max(idx[0], 0), E - 1);
  const float m = bias ? logits[(size_t)t * E + first] + bias[first] : logits[(size_t)t * E + first];
  float q[EPL], dq[EPL];
  float den = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    dq[i] = 0.f;
    bool chosen = false;
    for (int j = 0; j < k; ++j)
      if (idx[j] == e) {
        chosen = true;
        dq[i] = dg[(size_t)t * k + j];
      }
    bool in = false;
    if (e < E) {
      if (renorm) {
        in = chosen;
      } else if (presel > 0) {
        int rank = 0;
        for (int o = 0; o < E; ++o) {
          const float so = s_sc[w * E + o];
          rank += (so > sc[i]) || (so == sc[i] && o < e);
        }
        in = rank < presel;
      } else {
        in = true;
      }
    }
    q[i] = in ? expf(sc[i] - m) : 0.f;
    den += q[i];
  }
  den = wave_sum_f(den);
  float inner = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    q[i] = q[i] / den;
    inner += q[i] * dq[i];
  }
  inner = wave_sum_f(inner);
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      const float ds = q[i] * (dq[i] - inner);
      dz[(size_t)t * E + e] = ds;
      const __bf16 b = (__bf16)ds;
      dz_bf16[(size_t)t * E + e] = __builtin_bit_cast(uint16_t, b);
    }
  }
}

// d_bias: column sums of dz in a fixed order: 64-column x 128-row partials,
// then one thread per column adds the partials in row order.
constexpr int kBiasRows = 128;
constexpr int kBiasMaxChunks = 4096;
static int bias_chunk_rows(int T) { return T > kBiasRows * kBiasMaxChunks ? div_up(T, kBiasMaxChunks) : kBiasRows; }
__global__ __launch_bounds__(64) void bias_partial_kernel(const float* __restrict__ dz, int T, int E,
                                                          int chunk_rows, float* __restrict__ part) {
  const int e = blockIdx.x * 64 + threadIdx.x;
  const int r0 = blockIdx.y * chunk_rows;
  if (e >= E) return;
  float s = 0.f;
  const int r1 = min(T, r0 + chunk_rows);
  for (int t = r0; t < r1; ++t) s += dz[(size_t)t * E + e];
  part[(size_t)blockIdx.y * E + e] = s;
}
__global__ __launch_bounds__(256) void bias_final_kernel(const float* __restrict__ part, int chunks,
                                                         int E, float* __restrict__ db) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  float s = 0.f;
  for (int c = 0; c < chunks; ++c) s += part[(size_t)c * E + e];
  db[e] = s;
}

// ------------------------------------------------------------- dispatch backward
// One wave per token: dx[t] = sum_j dx_perm[p(t,j)] (+ dx_router[t]), fp32 in
// j order, one bf16 rounding.  KU > 0 (k <= KU): the k row bases are read
// once and the k loads of a vector are issued together; KU = 0: one row at a
// time.  The sum runs in the same order either way.
template <int KU>
__global__ __launch_bounds__(256) void unpermute_sum_kernel(const u32x4* __restrict__ dxp,
                                                            const int32_t* __restrict__ slot_of,
                                                            const u32x4* __restrict__ dxr,
                                                            u32x4* __restrict__ dx, int T, int k,
                                                            int nvec, int A) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  auto add = [](float* acc, const u32x4& r) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += bf16_lo(r[q]);
      acc[2 * q + 1] += bf16_hi(r[q]);
    }
  };
  size_t base[KU > 0 ? KU : 1];
  if constexpr (KU > 0) {
#pragma unroll
    for (int j = 0; j < KU; ++j)
      base[j] = j < k ? (size_t)min(max(slot_of[(size_t)t * k + j], 0), A - 1) * nvec : 0;
  }
  for (int v = lane; v < nvec; v += 64) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    if constexpr (KU > 0) {
      u32x4 r[KU];
#pragma unroll
      for (int j = 0; j < KU; ++j)
        if (j < k) r[j] = dxp[base[j] + v];
#pragma unroll
      for (int j = 0; j < KU; ++j)
        if (j < k) add(acc, r[j]);
    } else {
      for (int j = 0; j < k; ++j) {
        const int p = min(max(slot_of[(size_t)t * k + j], 0), A - 1);
        add(acc, dxp[(size_t)p * nvec + v]);
      }
    }
    if (dxr) add(acc, dxr[(size_t)t * nvec + v]);
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    dx[(size_t)t * nvec + v] = o;
  }
}

// ------------------------------------------------------------- launchers
hipError_t launch_combine_backward(const moe_config& c, const void* d_out, const void* y_perm,
                                   const int32_t* slot_of, const float* topk_w, void* d_y_perm,
                                   float* d_topk_w, hipStream_t st) {
  const int nvec = c.d / 8;
  const auto* dout = static_cast<const u32x4*>(d_out);
  const auto* y = static_cast<const u32x4*>(y_perm);
  auto* dy = static_cast<u32x4*>(d_y_perm);
  const int blocks = div_up(c.T, 4), A = c.T * c.k;
  if (nvec <= 64 * 4)
    combine_backward_kernel<4><<<blocks, 256, 0, st>>>(dout, y, slot_of, topk_w, dy, d_topk_w,
                                                       c.T, c.k, nvec, A);
  else if (nvec <= 64 * 16)
    combine_backward_kernel<16><<<blocks, 256, 0, st>>>(dout, y, slot_of, topk_w, dy, d_topk_w,
                                                        c.T, c.k, nvec, A);
  else
    combine_backward_kernel<0><<<blocks, 256, 0, st>>>(dout, y, slot_of, topk_w, dy, d_topk_w,
                                                       c.T, c.k, nvec, A);
  return hipGetLastError();
}

size_t ffn_backward_ws_bytes(const moe_config& c) {
  return 5 * (size_t)c.T * c.k * c.f * sizeof(uint16_t);  // a, u, dh / h, da | du
}

hipError_t launch_ffn_backward(const moe_config& c, const void* x_perm, const int32_t* offs,
                               const void* wg, const void* wu, const void* wd, const void* a_in,
                               const void* u_in, const void* packed_dh, const void* packed_dx,
                               const void* d_y_perm, void* d_x_perm, void* d_wg, void* d_wu,
                               void* d_wd, void* ws, hipStream_t st) {
  const int rows = c.T * c.k, d = c.d, f = c.f, E = c.E;
  const size_t af = (size_t)rows * f;
  uint16_t* a = static_cast<uint16_t*>(ws);  // recomputed a
  uint16_t* u = a + af;                       // recomputed u
  uint16_t* h = u + af;                       // dh, then h
  uint16_t* dadu = h + af;                    // [rows, 2 f]: da_r, du_r
  const auto* X = static_cast<const uint16_t*>(x_perm);
  const auto* dY = static_cast<const uint16_t*>(d_y_perm);
  const auto* Wg = static_cast<const uint16_t*>(wg);
  const auto* Wu = static_cast<const uint16_t*>(wu);
  const auto* Wd = static_cast<const uint16_t*>(wd);
  hipError_t err;
  if (rows == 0) {  // no rows: every weight gradient is zero
    if ((err = launch_wgrad(dY, d, h, f, offs, E, 0, d, f, static_cast<uint16_t*>(d_wd), f,
                            (long)d * f, st)) != hipSuccess)
      return err;
    if ((err = launch_wgrad(a, f, X, d, offs, E, 0, f, d, static_cast<uint16_t*>(d_wg), d,
                            (long)f * d, st)) != hipSuccess)
      return err;
    return launch_wgrad(u, f, X, d, offs, E, 0, f, d, static_cast<uint16_t*>(d_wu), d,
                        (long)f * d, st);
  }
  // the gate and up pre-activations: the training forward's, else recomputed
  // (the inference forward keeps only h)
  const uint16_t* a_src = static_cast<const uint16_t*>(a_in);
  const uint16_t* u_src = static_cast<const uint16_t*>(u_in);
  if (!a_src) {
    if ((err = launch_grouped_linear(c, X, offs, Wg, a, f, d, st)) != hipSuccess) return err;
    if ((err = launch_grouped_linear(c, X, offs, Wu, u, f, d, st)) != hipSuccess) return err;
    a_src = a;
    u_src = u;
  }
  // dh = dy Wd_e (Wd_e is [d, f]): on the packed image of W_d^T, else the dgrad
  if (packed_dh) {
    if ((err = launch_packed_linear(c, dY, offs, packed_dh, h, f, d, st)) != hipSuccess)
      return err;
  } else {
    GemmPart p{dY, Wd, d, f, (long)d * f, d};
    if ((err = launch_dgrad(&p, 1, offs, E, rows, f, h, f, st)) != hipSuccess) return err;
  }
  // h (over dh), da | du
  {
    const long nvec = (long)af / 8;
    swiglu_backward_kernel<<<div_up(nvec, 256), 256, 0, st>>>(
        reinterpret_cast<const u32x4*>(a_src), reinterpret_cast<const u32x4*>(u_src),
        reinterpret_cast<u32x4*>(h), reinterpret_cast<u32x4*>(dadu), (long)f / 8, nvec);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // dWd_e = dy_e^T h_e   [d, f]
  if ((err = launch_wgrad(dY, d, h, f, offs, E, rows, d, f, static_cast<uint16_t*>(d_wd), f,
                          (long)d * f, st)) != hipSuccess)
    return err;
  // dx = [da du] [Wg_e; Wu_e] (Wg_e, Wu_e are [f, d]): on the packed image of
  // [W_g; W_u]^T (k = 2 f), else the dgrad over two parts
  if (packed_dx) {
    if ((err = launch_packed_linear(c, dadu, offs, packed_dx, d_x_perm, d, 2 * f, st)) !=
        hipSuccess)
      return err;
  } else {
    GemmPart p[2] = {{dadu, Wg, 2L * f, d, (long)f * d, f},
                     {dadu + f, Wu, 2L * f, d, (long)f * d, f}};
    if ((err = launch_dgrad(p, 2, offs, E, rows, d, static_cast<uint16_t*>(d_x_perm), d, st)) !=
        hipSuccess)
      return err;
  }
  // dWg_e = da_e^T x_e, dWu_e = du_e^T x_e   [f, d]
  if ((err = launch_wgrad(dadu, 2L * f, X, d, offs, E, rows, f, d, static_cast<uint16_t*>(d_wg),
                          d, (long)f * d, st)) != hipSuccess)
    return err;
  return launch_wgrad(dadu + f, 2L * f, X, d, offs, E, rows, f, d,
                      static_cast<uint16_t*>(d_wu), d, (long)f * d, st);
}

// dWr = dz^T x has only E output rows and a reduction over all T tokens:
// its 128 x 128 tiles are few (E = 16, d = 5120: 40), each with a long k
// loop.  The reduction is split over S row segments so that S times the
// tiles fill the chip about twice; each segment's tile writes float32
// partial sums and router_split_sum_kernel adds the S partials (segment
// order, float32) and rounds once to bf16.  S = 1 keeps the direct path.
constexpr int kRouterMaxSplit = 16;
constexpr int kRouterMinSegRows = 64;
static int router_wgrad_split(const moe_config& c) {
  const long tiles = (long)div_up(c.E, 128) * div_up(c.d, 128);
  const long want = div_up(2L * kCUs, tiles);
  const long cap = std::min<long>(kRouterMaxSplit, c.T / kRouterMinSegRows);
  return (int)std::max<long>(1, std::min(want, cap));
}

__global__ void split_offsets_kernel(int32_t* __restrict__ offs, int S, int T) {
  const int s = threadIdx.x;
  if (s <= S) offs[s] = (int)((long)s * T / S);
}

// out[i] = bf16(part[0][i] + part[1][i] + ... + part[S-1][i]), 4 per thread.
__global__ __launch_bounds__(256) void router_split_sum_kernel(const float4* __restrict__ part,
                                                               int S, long n4,
                                                               u32x2* __restrict__ out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  float4 acc = part[i];
  for (int s = 1; s < S; ++s) {
    const float4 v = part[(long)s * n4 + i];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  u32x2 o;
  o.x = pack_bf16x2(acc.x, acc.y);
  o.y = pack_bf16x2(acc.z, acc.w);
  out[i] = o;
}

static size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// dz (bf16) | {0, T} | d_bias chunk partials | split offsets | dWr partials
size_t route_backward_ws_bytes(const moe_config& c) {
  const size_t dzb = round256((size_t)c.T * c.E * sizeof(uint16_t));
  const int T1 = c.T > 0 ? c.T : 1;
  const size_t part = round256((size_t)div_up(T1, bias_chunk_rows(T1)) * c.E * sizeof(float));
  const int S = router_wgrad_split(c);
  const size_t split = S > 1 ? 256 + (size_t)S * c.E * c.d * sizeof(float) : 0;
  return dzb + 256 + part + split;
}

hipError_t launch_route_backward(const moe_config& c, const void* x, const void* w_router,
                                 const float* logits, const float* bias, const int32_t* topk_idx,
                                 const float* d_topk_w, float* d_logits, void* d_x_router,
                                 void* d_w_router, float* d_bias, void* ws, hipStream_t st) {
  const int T = c.T, E = c.E, d = c.d;
  char* wsb = static_cast<char*>(ws);
  uint16_t* dzb = reinterpret_cast<uint16_t*>(wsb);
  const size_t dzb_bytes = ((size_t)T * E * sizeof(uint16_t) + 255) / 256 * 256;
  int32_t* offs = reinterpret_cast<int32_t*>(wsb + dzb_bytes);  // {0, T}
  float* part = reinterpret_cast<float*>(wsb + dzb_bytes + 256);
  const int T1 = T > 0 ? T : 1;
  char* split_base =
      wsb + dzb_bytes + 256 + round256((size_t)div_up(T1, bias_chunk_rows(T1)) * E * sizeof(float));
  hipError_t err;
  if (T > 0) {
    const dim3 grid(div_up(T, 4));
    const size_t lds = (!c.renorm && c.presel > 0) ? 4 * (size_t)E * sizeof(float) : 0;
    if (E <= 64)
      gates_backward_kernel<1><<<grid, 256, lds, st>>>(logits, bias, topk_idx, d_topk_w, T, E, c.k,
                                                       c.presel, c.renorm, d_logits, dzb);
    else if (E <= 256)
      gates_backward_kernel<4><<<grid, 256, lds, st>>>(logits, bias, topk_idx, d_topk_w, T, E, c.k,
                                                       c.presel, c.renorm, d_logits, dzb);
    else
      gates_backward_kernel<16><<<grid, 256, lds, st>>>(logits, bias, topk_idx, d_topk_w, T, E,
                                                        c.k, c.presel, c.renorm, d_logits, dzb);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (d_bias) {
    const int rows_per = bias_chunk_rows(T);
    const int chunks = div_up(T, rows_per);
    if (chunks > 0)
      bias_partial_kernel<<<dim3(div_up(E, 64), chunks), 64, 0, st>>>(d_logits, T, E, rows_per,
                                                                      part);
    bias_final_kernel<<<div_up(E, 256), 256, 0, st>>>(part, chunks, E, d_bias);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if ((err = launch_fill_i32(offs, 1, 0, st)) != hipSuccess) return err;
  if ((err = launch_fill_i32(offs + 1, 1, T, st)) != hipSuccess) return err;
  // dx_router = dz Wr   (Wr is [E, d]: the [K, N] weights of one group)
  {
    GemmPart p{dzb, static_cast<const uint16_t*>(w_router), E, d, 0, E};
    if ((err = launch_dgrad(&p, 1, offs, 1, T, d, static_cast<uint16_t*>(d_x_router), d, st)) !=
        hipSuccess)
      return err;
  }
  // dWr = dz^T x   [E, d]
  const int S = router_wgrad_split(c);
  if (S == 1)
    return launch_wgrad(dzb, E, static_cast<const uint16_t*>(x), d, offs, 1, T, E, d,
                        static_cast<uint16_t*>(d_w_router), d, 0, st);
  int32_t* soffs = reinterpret_cast<int32_t*>(split_base);  // S + 1 <= 64 entries
  float* rpart = reinterpret_cast<float*>(split_base + 256);
  split_offsets_kernel<<<1, 64, 0, st>>>(soffs, S, T);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int mt = div_up(E, 128), nt = div_up(d, 128);
  wgrad_dma_kernel<128, 128, true><<<S * mt * nt, 256, 0, st>>>(
      dzb, E, static_cast<const uint16_t*>(x), d, soffs, S, T, E, d, mt, nt, rpart, d,
      (long)E * d);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const long n4 = (long)E * d / 4;
  router_split_sum_kernel<<<div_up(n4, 256), 256, 0, st>>>(
      reinterpret_cast<const float4*>(rpart), S, n4, static_cast<u32x2*>(d_w_router));
  return hipGetLastError();
}

hipError_t launch_unpermute_backward(const moe_config& c, const void* d_x_perm,
                                     const int32_t* slot_of, const void* d_x_router, void* d_x,
                                     hipStream_t st) {
  const int nvec = c.d / 8;
  const auto* dxp = static_cast<const u32x4*>(d_x_perm);
  const auto* dxr = static_cast<const u32x4*>(d_x_router);
  auto* dx = static_cast<u32x4*>(d_x);
  const int blocks = div_up(c.T, 4), A = c.T * c.k;
  // the batched loads pay off for k <= 2 (T1024-E8: 29 -> 17 us); at k = 8
  // (T8192-E256) they measured 5 % slower than one row at a time
  if (c.k <= 2)
    unpermute_sum_kernel<2><<<blocks, 256, 0, st>>>(dxp, slot_of, dxr, dx, c.T, c.k, nvec, A);
  else
    unpermute_sum_kernel<0><<<blocks, 256, 0, st>>>(dxp, slot_of, dxr, dx, c.T, c.k, nvec, A);
  return hipGetLastError();
}

}  // namespace moe
