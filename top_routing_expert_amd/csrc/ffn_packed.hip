// Grouped expert FFN on pre-packed expert weights (bf16).
//
// Same computation as the row-major path: for each expert e, the rows
// [off[e], off[e+1]) of the permuted activations go through
//   h = SiLU(X Wg^T) * (X Wu^T)   (gate_up)   and   y = h Wd^T   (down).
// Pages: [V4-overlap] Waved-EP section (expert compute = L1 + Act + L2);
// [EP-V4] §5.2 (expert weights contiguous and in expert-ID order: the packed
// image keeps that order, so a sub-table of experts is still a plain offset).
//
// Why a packed image.  For the token counts an expert sees in a layer
// (hundreds of rows), the grouped GEMM streams every weight byte from HBM
// once while the tokens stay in L2.  Staging the weights through LDS costs
// LDS bandwidth on the write and on the fragment reads of every wave, and the
// LDS ring bounds how far ahead the weight stream can run.  Packed once into
// MFMA fragment order, the weights go straight from HBM into the registers of
// the one wave that uses them: each wave instruction reads 1 KB of
// consecutive bytes, and a register queue keeps 8 k-steps (16 KB per wave,
// 64 KB per CU) in flight.  Only the tokens, shared by all four waves, pass
// through LDS.
//
// Packed image of one weight set, per expert (experts back to back):
//   [slab][wave 0..3][k-step 0..Kp/16-1][fragment 0..1][lane 0..63][8 bf16]
// Kp = K rounded up to 128 (zero padded).  Lane l of fragment (slab, w, i)
// at k-step s holds row (l & 31) of the fragment and k = 16 s + 8 (l >> 5)
// .. +7, which is the MFMA 32x32x16 A-operand layout.
//   gate_up: a slab is 128 output features; fragment (w, i) has rows 0..15 =
//     W_gate rows F..F+15 and rows 16..31 = W_up rows F..F+15 with
//     F = 128 slab + 32 w + 16 i, so gate and up of a feature meet in the
//     same lane (accumulator registers r and r + 8) and SiLU(g)*u is applied
//     in registers.
//   down: a slab is 256 output features; fragment (w, i) has rows
//     F..F+31 of W_down with F = 256 slab + 64 w + 32 i.
//   Rows past the last feature are zero.
//
// Kernel (persistent, one block of 4 waves per CU, 256 accumulators per wave):
//  * tile = one slab x up to 256 token rows of one expert; wave w owns two
//    32-row weight fragments (64 rows) against all token fragments, so every
//    weight byte is used by exactly one wave.
//  * k loop in iterations of 128 (8 MFMA k-steps).  Weight fragments for
//    k-step s+8 are loaded into the register slot of k-step s right after the
//    MFMAs that use it.  Token rows pass through a ring of four 64-wide k
//    half-stages in LDS (rows of 128 bytes, 16-byte pieces XOR-swizzled with
//    (row >> 1) & 7 so the 16 lanes of a 16-byte read hit 16 bank groups):
//    each half-stage is loaded into registers one half-stage ahead and written
//    two ahead; one barrier per half-stage.
//  * Operands are read through buffer resources (one address register per
//    stream); all loads are compiler-visible, so its vmcnt waits are exact.
//  * The main loop is specialised on the number of 32-token fragments that
//    hold rows; padded token rows read a clamped (real) row and are not
//    stored; padded k reads zeros.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "common.h"
#include "tiles.h"

namespace moe {

constexpr int kPkIterK = 128;  // k per main-loop iteration
constexpr int kPkSteps = 8;    // MFMA k-steps (16 wide) per iteration
// Word 3 of a raw (untyped, unswizzled) buffer resource on gfx950.
constexpr int kBufferFlags = 0x00020000;

// Features per slab and packed geometry of one weight set.
PackGeom pack_geom(int features, int K, bool gated) {
  PackGeom g;
  g.slab_features = gated ? 128 : 256;
  g.slabs = div_up(features, g.slab_features);
  g.kp = div_up(K, kPkIterK) * kPkIterK;
  g.expert_elems = (size_t)g.slabs * 256 * g.kp;
  return g;
}

// One thread per 16-byte piece of the packed image.
template <bool GATED>
__global__ void pack_weights_kernel(const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1,
                                    u32x4* __restrict__ dst, int F, int K, int slabs, int kp,
                                    size_t total) {
  const int nks = kp / 16;
  for (size_t p = blockIdx.x * (size_t)blockDim.x + threadIdx.x; p < total;
       p += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(p & 63);
    size_t r = p >> 6;
    const int i = (int)(r & 1);
    r >>= 1;
    const int ks = (int)(r % nks);
    r /= nks;
    const int w = (int)(r & 3);
    r >>= 2;
    const int slab = (int)(r % slabs);
    const size_t e = r / slabs;
    const int row = lane & 31;
    const int k = ks * 16 + 8 * (lane >> 5);
    int feat;
    const uint16_t* base;
    if (GATED) {
      feat = slab * 128 + w * 32 + i * 16 + (row & 15);
      base = row < 16 ? w0 : w1;
    } else {
      feat = slab * 256 + w * 64 + i * 32 + row;
      base = w0;
    }
    u32x4 v = {0u, 0u, 0u, 0u};
    if (feat < F && k < K) v = *reinterpret_cast<const u32x4*>(base + (e * F + feat) * (size_t)K + k);
    dst[p] = v;
  }
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 (compile-time index).
template <int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>()), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<N>(f, std::make_integer_sequence<int, N>());
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// JMAX: 32-token fragments per block tile (tile = 32 JMAX tokens).
//
// Persistent: the grid holds one block per CU (a multiple of 8) and every
// block walks its own list of tiles.  Tiles go out in rounds of one tile per
// block; inside a round, consecutive tiles go to the blocks of one XCD (the
// hardware hands blocks to XCDs round-robin, block b to XCD b % 8), so the
// tiles running at once on an XCD are neighbours in the tile order and share
// weight and token rows in its L2; every other round runs backwards, which
// evens out the per-block totals when tiles differ in size.  A grid of one
// block per tile would be dispatched in block order, and an XCD whose tiles
// run long would hold back the dispatch of every other XCD.
template <bool GATED, int JMAX, int OCC>
__global__ __launch_bounds__(256, OCC) void grouped_gemm_packed_kernel(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ offs,
    const u32x4* __restrict__ wp, uint16_t* __restrict__ out, int E, int N, int K, int rows,
    int slabs, int band) {
  constexpr int TM = 32 * JMAX;
  // k-steps of weight fragments in flight per wave: 8 with one block per CU;
  // 4 with two, whose other block's waves cover the rest of the latency
  constexpr int WQ = (OCC == 1 && JMAX <= 8) ? kPkSteps : kPkSteps / 2;
  constexpr int TN = GATED ? 128 : 256;  // output features per slab
  constexpr int HALF = TM * 8;           // 16-byte pieces of one 64-wide k half-stage
  // LDS ring of 64-wide k half-stages: four slots, three for 320-row tiles
  constexpr int NSLOT = JMAX > 8 ? 3 : 4;
  static_assert(JMAX <= 10, "at most 10 token fragments per tile");
  __shared__ u32x4 tok[NSLOT * HALF];
  __shared__ int s_tile[4];

  const int G = (int)gridDim.x;
  const int qp = (G >> 3) * (int)(blockIdx.x & 7) + (int)(blockIdx.x >> 3);
  __shared__ int s_total;
  if (threadIdx.x < 64) {
    const int n = count_row_tiles<TM>(offs, E, rows, (int)threadIdx.x) * slabs;
    if (threadIdx.x == 0) s_total = n;
  }
  for (int round = 0;; ++round) {
  // Per-tile state is recomputed every round: values live across the loop
  // would push the main loop's register allocation past the register file.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));  // keep the compiler from hoisting lane state out of the loop
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wave == 0) {  // s_total and s_tile: written and read in order by this one wave
    const int L = round * G + ((round & 1) ? G - 1 - qp : qp);
    if (lane == 0) s_tile[0] = -1;
    if (L < s_total) locate_tile<TM>(offs, E, rows, slabs, band, L, lane, s_tile);
  }
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(s_tile[0]);
  if (e < 0) break;  // block-uniform; later rounds only hold larger tile numbers
  const int kp = (K + kPkIterK - 1) / kPkIterK * kPkIterK;
  const int nit = kp / kPkIterK;
  const uint32_t wl = (uint32_t)lane * 16u;
  // the activations as one buffer resource: rows * K * 2 < 2^32 bytes
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(act), (short)0, (int)((uint32_t)rows * (uint32_t)K * 2u), kBufferFlags);

  // Token half-stage h = k range [64 h, 64 h + 64) of the tile's rows: LDS
  // rows of 128 bytes, 16-byte piece q of row r at q ^ ((r >> 1) & 7), so the
  // 16 lanes served together by a 16-byte LDS read (16 consecutive rows, one
  // piece) hit 16 different bank groups.  Load chunk c covers tile rows
  // 32c..32c+31; this lane takes row 32c + 8 wave + lane/8, piece lane & 7.
  const int tq = lane & 7, trow = 8 * wave + (lane >> 3);
  const int tpos = trow * 8 + (tq ^ ((trow >> 1) & 7));  // LDS piece in chunk 0
  // fragment reads: token row 32 j + (lane & 31), piece (2 u' + lk) ^ (row >> 1 & 7)
  const int lk = lane >> 5, bbase = (lane & 31) * 8, bsw = (lane >> 1) & 7;
  const int row0 = __builtin_amdgcn_readfirstlane(s_tile[1]);
  const int row_end = __builtin_amdgcn_readfirstlane(s_tile[2]);
  const int slab = __builtin_amdgcn_readfirstlane(s_tile[3]);
  const int nrow = min(row_end - row0, TM);
  const int jn = (nrow + 31) >> 5;  // live token fragments, 1..JMAX
  // This wave's weight stream as a buffer resource (wave-uniform base and
  // size): a load is one VGPR offset (the lane's 16 bytes) plus a uniform
  // offset (fragment i of k-step s), so the stream costs no address registers.
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u32x4*>(wp + (((size_t)e * slabs + slab) * 4 + wave) * ((size_t)(kp / 16) * 128)),
      (short)0, (kp / 16) * 2048, kBufferFlags);
  auto wload = [&](int s, int i) -> u32x4 {  // fragment i of k-step s
    return __builtin_amdgcn_raw_buffer_load_b128(wrsrc, (int)wl, s * 2048 + i * 1024, 0);
  };

  auto run = [&](auto jn_c) {
    constexpr int JN = decltype(jn_c)::value;
    // Load chunk c covers tile rows 32c..32c+31.  Only the last chunk can
    // reach past the expert's rows; it reads a clamped (real) row instead.
    // The other chunks are this lane's row plus a uniform stride.
    const uint32_t toff0 = ((uint32_t)(row0 + trow) * (uint32_t)K + 8u * tq) * 2u;
    const uint32_t tofl =
        ((uint32_t)(row0 + min(32 * (JN - 1) + trow, nrow - 1)) * (uint32_t)K + 8u * tq) * 2u;
    const int cstride = 64 * K;  // bytes of 32 rows
    // Half-stages past K (K % 128 == 64) re-read the last real one: their
    // weights are zero in the packed image, so they add exact zeros.
    const int hlast = K / 64 - 1;
    auto load_chunk = [&](int h, int c) -> u32x4 {
      const int hb = min(h, hlast) * 128;
      if (c == JN - 1) return __builtin_amdgcn_raw_buffer_load_b128(arsrc, (int)tofl, hb, 0);
      return __builtin_amdgcn_raw_buffer_load_b128(arsrc, (int)toff0, hb + c * cstride, 0);
    };
    auto slot = [&](int h) -> u32x4* { return tok + (h % NSLOT) * HALF; };

    // Pipeline.  Half-stage h (k range [64 h, 64 h + 64)) lives in LDS slot
    // h % NSLOT.  While the MFMAs of half-stage h run, the staged registers
    // sg (half-stage h+2, loaded during h-1) are written to slot h+2 and sg
    // is refilled with h+3, a quarter of the chunks per k-step, so every load
    // has four k-steps before its LDS write.  Slot h+2 was last read during
    // h-1 (three slots) or h-2 (four), and a barrier ends every half-stage.
    // The B fragment of token fragment j for the next k-step is read into the
    // same registers right after the last MFMA that uses it, so the reads of
    // one k-step overlap the MFMAs of the one before.  Weight fragment i of
    // k-step s+WQ is loaded into wq slot s % WQ right after its last MFMA.
    u32x4 wq[WQ][2];
    u32x4 sg[JN];
    u32x4 bq[JN];
    // prologue, issued in the steady state's order: half-stages 0 and 1 (to
    // LDS now), k-steps 0..3, then half-stage 2 interleaved with k-steps 4..7
    u32x4 s0[JN], s1[JN];
#pragma unroll
    for (int c = 0; c < JN; ++c) s0[c] = load_chunk(0, c);
#pragma unroll
    for (int c = 0; c < JN; ++c) s1[c] = load_chunk(1, c);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int i = 0; i < 2; ++i) wq[u][i] = wload(u, i);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = 4; u < 8; ++u) {
#pragma unroll
      for (int c = JN * (u - 4) / 4; c < JN * (u - 3) / 4; ++c)
        sg[c] = load_chunk(2, c);  // clamped: valid even when nit == 1
      __builtin_amdgcn_sched_barrier(0);
      if (u < WQ) {
#pragma unroll
        for (int i = 0; i < 2; ++i) wq[u][i] = wload(u, i);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int c = 0; c < JN; ++c) tok[tpos + 256 * c] = s0[c];
#pragma unroll
    for (int c = 0; c < JN; ++c) tok[HALF + tpos + 256 * c] = s1[c];
    lds_barrier();
    {
      const int q = lk ^ bsw;
#pragma unroll
      for (int j = 0; j < JN; ++j) bq[j] = tok[bbase + 256 * j + q];
    }
    // the accumulators come to life only now, after the prologue's staging
    // registers are dead (both together would not fit the register file)
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc[2][JN];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < JN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // VAR 0: full iteration; 1: the one before the last (no load of
    // half-stage 2t+4); 2: the last (no loads, no LDS writes, no barrier).
    auto iter = [&](int t, auto var_c) {
      constexpr int VAR = decltype(var_c)::value;
      __builtin_amdgcn_sched_barrier(0);
      static_for<kPkSteps>([&](auto u_c) {
        constexpr int u = decltype(u_c)::value;
        constexpr int ph = u >> 2, uu = u & 3;  // half of the iteration, k-step in it
        constexpr int c_lo = JN * uu / 4, c_hi = JN * (uu + 1) / 4;
        constexpr int n_chunk = c_hi - c_lo;
        constexpr bool WRITE = VAR < 2;
        constexpr bool LOAD = VAR == 0 || (VAR == 1 && ph == 0);
        constexpr bool NEXT_B = u < 7 || VAR < 2;
        constexpr bool WLOAD = VAR < 2 || u + WQ < kPkSteps;  // k-step s+WQ still in range
        const int h = 2 * t + ph;
#pragma unroll
        for (int c = c_lo; c < c_hi; ++c) {
          if (WRITE) slot(h + 2)[tpos + 256 * c] = sg[c];
          if (LOAD) sg[c] = load_chunk(h + 3, c);
        }
        // next k-step's B fragments: slot and piece
        const u32x4* nb_slot = slot(u < 7 ? h + (uu == 3 ? 1 : 0) : 2 * t + 2);
        const int nq = (2 * ((u + 1) & 3) + lk) ^ bsw;
        // i-major MFMA order: weight fragment 0 is free after the first JN
        // MFMAs, fragment 1 and every B fragment after their last use
#pragma unroll
        for (int j = 0; j < JN; ++j)
          acc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(wq[u % WQ][0]),
                                                              as_bf16x8(bq[j]), acc[0][j], 0, 0, 0);
        if (WLOAD) wq[u % WQ][0] = wload(t * kPkSteps + u + WQ, 0);
#pragma unroll
        for (int j = 0; j < JN; ++j) {
          acc[1][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(wq[u % WQ][1]),
                                                              as_bf16x8(bq[j]), acc[1][j], 0, 0, 0);
          if (NEXT_B) bq[j] = nb_slot[bbase + 256 * j + nq];
        }
        if (WLOAD) wq[u % WQ][1] = wload(t * kPkSteps + u + WQ, 1);
        // Issue order: the staged LDS writes first (their loads are four
        // k-steps old), the token loads among the first MFMAs, then each B
        // fragment read after its last MFMA.
        constexpr int n_dsw = WRITE ? n_chunk : 0;
        constexpr int n_tl = LOAD ? n_chunk : 0;
        if (n_dsw > 0) __builtin_amdgcn_sched_group_barrier(0x200, n_dsw, 0);
        static_for<n_tl>([&](auto) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        });
        __builtin_amdgcn_sched_group_barrier(0x008, JN - n_tl, 0);
        if (WLOAD) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        static_for<JN>([&](auto) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (NEXT_B) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        });
        if (WLOAD) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (uu == 3 && VAR < 2) {
          lds_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
      });
    };
    int t = 0;
    for (; t + 2 < nit; ++t) iter(t, std::integral_constant<int, 0>());
    if (nit >= 2) {
      iter(t, std::integral_constant<int, 1>());
      ++t;
    }
    iter(t, std::integral_constant<int, 2>());

    // epilogue: acc[i][j][4 g + r] = C[fragment row 8 g + 4 lk + r][token lane & 31]
    const int nb = slab * TN + wave * (TN / 4);
#pragma unroll
    for (int j = 0; j < JN; ++j) {
      const int p = row0 + 32 * j + (lane & 31);
      if (p >= row_end) continue;
      uint16_t* orow = out + (size_t)p * N;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (GATED) {
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const int n = nb + 16 * i + 8 * g + 4 * lk;
            if (n >= N) continue;
            float hv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float gt = acc[i][j][4 * g + r], up = acc[i][j][4 * g + 8 + r];
              hv[r] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
            }
            u32x2 pk;
            pk.x = pack_bf16x2(hv[0], hv[1]);
            pk.y = pack_bf16x2(hv[2], hv[3]);
            *reinterpret_cast<u32x2*>(orow + n) = pk;
          }
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = nb + 32 * i + 8 * g + 4 * lk;
            if (n >= N) continue;
            u32x2 pk;
            pk.x = pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
            pk.y = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
            *reinterpret_cast<u32x2*>(orow + n) = pk;
          }
        }
      }
    }
  };
  switch (jn) {
    case 1: run(std::integral_constant<int, 1>()); break;
    case 2: run(std::integral_constant<int, (2 < JMAX ? 2 : JMAX)>()); break;
    case 3: run(std::integral_constant<int, (3 < JMAX ? 3 : JMAX)>()); break;
    case 4: run(std::integral_constant<int, (4 < JMAX ? 4 : JMAX)>()); break;
    case 5: run(std::integral_constant<int, (5 < JMAX ? 5 : JMAX)>()); break;
    case 6: run(std::integral_constant<int, (6 < JMAX ? 6 : JMAX)>()); break;
    case 7: run(std::integral_constant<int, (7 < JMAX ? 7 : JMAX)>()); break;
    case 8: run(std::integral_constant<int, (8 < JMAX ? 8 : JMAX)>()); break;
    case 9: run(std::integral_constant<int, (9 < JMAX ? 9 : JMAX)>()); break;
    default: run(std::integral_constant<int, JMAX>()); break;
  }
  // every wave is done with the LDS ring and s_tile before the next tile
  __syncthreads();
  }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_pack_weights(const moe_config& c, const void* wg, const void* wu, const void* wd,
                               void* pgu, void* pd, hipStream_t st) {
  auto pack = [&](bool gated, const void* a, const void* b, void* dst, int F, int K) {
    const PackGeom g = pack_geom(F, K, gated);
    const size_t total = (size_t)c.E * g.expert_elems / 8;
    const int blocks = (int)std::min<size_t>((total + 255) / 256, (size_t)1 << 20);
    if (gated)
      pack_weights_kernel<true><<<blocks, 256, 0, st>>>(static_cast<const uint16_t*>(a),
                                                         static_cast<const uint16_t*>(b),
                                                         static_cast<u32x4*>(dst), F, K, g.slabs,
                                                         g.kp, total);
    else
      pack_weights_kernel<false><<<blocks, 256, 0, st>>>(static_cast<const uint16_t*>(a), nullptr,
                                                          static_cast<u32x4*>(dst), F, K, g.slabs,
                                                          g.kp, total);
    return hipGetLastError();
  };
  if (pgu) {
    hipError_t e = pack(true, wg, wu, pgu, c.f, c.d);
    if (e != hipSuccess) return e;
  }
  if (pd) return pack(false, wd, nullptr, pd, c.d, c.f);
  return hipSuccess;
}

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

#ifndef PK_JMAX_GU
#define PK_JMAX_GU 8
#endif
#ifndef PK_JMAX_DN
#define PK_JMAX_DN 8
#endif
template <bool GATED, int JMAX>
static hipError_t launch_packed_j(const moe_config& c, const void* act, const int32_t* offs,
                                  const void* wp, void* out, hipStream_t st) {
  constexpr int OCC = JMAX <= 4 ? 2 : 1;  // blocks per CU
  const long rows = (long)c.T * c.k;
  const int N = GATED ? c.f : c.d, K = GATED ? c.d : c.f;
  const PackGeom g = pack_geom(N, K, GATED);
  // OCC blocks per CU (never more blocks than the worst-case tile count)
  const long worst = (long)g.slabs * worst_row_tiles(rows, c.E, 32 * JMAX);
  const long cap = ((long)device_cus() * OCC + 7) / 8 * 8;
  const int blocks = (int)std::min(cap, (worst + 7) / 8 * 8);
  grouped_gemm_packed_kernel<GATED, JMAX, OCC><<<blocks, 256, 0, st>>>(
      static_cast<const uint16_t*>(act), offs, static_cast<const u32x4*>(wp),
      static_cast<uint16_t*>(out), c.E, N, K, (int)rows, g.slabs, 8);
  return hipGetLastError();
}

template <bool GATED>
static hipError_t launch_packed(const moe_config& c, const void* act, const int32_t* offs,
                                const void* wp, void* out, hipStream_t st) {
  return launch_packed_j<GATED, GATED ? PK_JMAX_GU : PK_JMAX_DN>(c, act, offs, wp, out, st);
}

hipError_t launch_ffn_gate_up_packed(const moe_config& c, const void* x_perm, const int32_t* offs,
                                     const void* pgu, void* h, hipStream_t st) {
  return launch_packed<true>(c, x_perm, offs, pgu, h, st);
}

hipError_t launch_ffn_down_packed(const moe_config& c, const void* h, const int32_t* offs,
                                  const void* pd, void* y, hipStream_t st) {
  return launch_packed<false>(c, h, offs, pd, y, st);
}

}  // namespace moe
