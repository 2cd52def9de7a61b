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
// Kernel (one block of 4 waves per CU, 256 accumulators per wave):
//  * block tile = one slab x up to 256 tokens of one expert; wave w owns two
//    32-row weight fragments (64 rows) against all token fragments, so every
//    weight byte is used by exactly one wave.
//  * k loop in iterations of 128 (8 MFMA k-steps).  Weight fragments for
//    k-step s+8 are loaded into the register slot of k-step s right after its
//    MFMAs.  The next 128-wide token stage is loaded into registers during
//    k-steps 0..3 and written to the other LDS buffer during k-steps 4..7
//    (LDS rows of 256 bytes, 16-byte pieces XOR-swizzled with row & 15); one
//    barrier per iteration.
//  * All loads are ordinary compiler-visible loads, so the compiler's own
//    vmcnt waits are exact.
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
template <bool GATED, int JMAX>
__global__ __launch_bounds__(256, 1) void grouped_gemm_packed_kernel(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ offs,
    const u32x4* __restrict__ wp, uint16_t* __restrict__ out, int E, int N, int K, int rows,
    int slabs, int band) {
  constexpr int TM = 32 * JMAX;
  constexpr int TN = GATED ? 128 : 256;  // output features per slab
  constexpr int HALF = TM * 8;           // 16-byte pieces of one 64-wide k half-stage
  static_assert(JMAX <= 8, "two staging chunks per k-step cover at most 8 fragments");
  __shared__ u32x4 tok[4 * HALF];        // ring of four 64-wide k half-stages
  __shared__ int s_tile[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wave == 0) place_tile<TM>(offs, E, rows, slabs, band, lane, s_tile);
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(s_tile[0]);
  if (e < 0) return;  // block-uniform
  const int row0 = __builtin_amdgcn_readfirstlane(s_tile[1]);
  const int row_end = __builtin_amdgcn_readfirstlane(s_tile[2]);
  const int slab = __builtin_amdgcn_readfirstlane(s_tile[3]);
  const int nrow = min(row_end - row0, TM);
  const int jn = (nrow + 31) >> 5;  // live token fragments, 1..JMAX
  const int kp = (K + kPkIterK - 1) / kPkIterK * kPkIterK;
  const int nit = kp / kPkIterK;
  // this wave's weight stream (wave-uniform base) and the lane's byte offset in it
  const char* __restrict__ wbase = reinterpret_cast<const char*>(
      wp + (((size_t)e * slabs + slab) * 4 + wave) * ((size_t)(kp / 16) * 128));
  const uint32_t wl = (uint32_t)lane * 16u;
  auto wload = [&](int s, int i) -> u32x4 {  // fragment i of k-step s
    return *reinterpret_cast<const u32x4*>(wbase + (size_t)(s * 2 + i) * 1024 + wl);
  };
  const char* __restrict__ abase = reinterpret_cast<const char*>(act);

  // Token half-stage h = k range [64 h, 64 h + 64) of the tile's rows: LDS
  // rows of 128 bytes, 16-byte piece q of row r at q ^ (r & 7).  Load chunk c
  // covers tile rows 32c..32c+31; this lane takes row 32c + 8 wave + lane/8,
  // piece lane & 7.
  const int tq = lane & 7, trow = 8 * wave + (lane >> 3);
  const int tpos = trow * 8 + (tq ^ (trow & 7));  // LDS piece in chunk 0
  // fragment reads: token row 32 j + (lane & 31), piece (2 u' + lk) ^ (lane & 7)
  const int lk = lane >> 5, bbase = (lane & 31) * 8, bsw = lane & 7;

  auto run = [&](auto jn_c) {
    constexpr int JN = decltype(jn_c)::value;
    // byte offset of each load chunk's row (clamped to the tile's last row)
    uint32_t toff[JN];
#pragma unroll
    for (int c = 0; c < JN; ++c)
      toff[c] = ((uint32_t)(row0 + min(32 * c + trow, nrow - 1)) * (uint32_t)K + 8u * tq) * 2u;
    // Half-stages past K (K % 128 == 64) re-read the last real one: their
    // weights are zero in the packed image, so they add exact zeros.
    const int hlast = K / 64 - 1;
    auto load_chunk = [&](int h, int c) -> u32x4 {
      return *reinterpret_cast<const u32x4*>(abase + (size_t)min(h, hlast) * 128 + toff[c]);
    };
    // B fragments of k-step u of iteration t (LDS slot of its half-stage)
    auto read_b = [&](int t, int u, u32x4(&b)[JN]) {
      const u32x4* cur = tok + ((2 * t + (u >> 2)) & 3) * HALF;
      const int q = (2 * (u & 3) + lk) ^ bsw;
#pragma unroll
      for (int j = 0; j < JN; ++j) b[j] = cur[bbase + 256 * j + q];
    };

    f32x16 acc[2][JN];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < JN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Pipeline.  Half-stage h (k range [64 h, 64 h + 64)) lives in LDS slot
    // h % 4.  While the MFMAs of half-stage h run, the staged registers sg
    // (half-stage h+2, loaded during h-1) are written to slot h+2 and sg is
    // refilled with h+3, two chunks per k-step, so every load has four
    // k-steps before its LDS write.  A barrier ends each half-stage; because
    // writes run two half-stages ahead, the B fragments of the first k-step
    // after a barrier are already read before it.  Weight fragments of k-step
    // s+8 are loaded into wq slot s % 8 right after the MFMAs of k-step s.
    u32x4 wq[kPkSteps][2];
    u32x4 sg[JN];
    u32x4 bA[JN], bB[JN];
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
      for (int c = 2 * (u - 4); c < 2 * (u - 4) + 2; ++c)
        if (c < JN) sg[c] = load_chunk(2, c);  // clamped: valid even when nit == 1
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2; ++i) wq[u][i] = wload(u, i);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int c = 0; c < JN; ++c) tok[tpos + 256 * c] = s0[c];
#pragma unroll
    for (int c = 0; c < JN; ++c) tok[HALF + tpos + 256 * c] = s1[c];
    lds_barrier();
    read_b(0, 0, bA);

    // VAR 0: full iteration; 1: the one before the last (no load of
    // half-stage 2t+4); 2: the last (no loads, no LDS writes, no barrier).
    auto iter = [&](int t, auto var_c) {
      constexpr int VAR = decltype(var_c)::value;
      __builtin_amdgcn_sched_barrier(0);
      static_for<kPkSteps>([&](auto u_c) {
        constexpr int u = decltype(u_c)::value;
        constexpr int ph = u >> 2, uu = u & 3;  // half of the iteration, k-step in it
        constexpr int n_chunk = (2 * uu + 2 <= JN) ? 2 : (2 * uu < JN ? JN - 2 * uu : 0);
        constexpr bool WRITE = VAR < 2;
        constexpr bool LOAD = VAR == 0 || (VAR == 1 && ph == 0);
        constexpr int n_dsw = WRITE ? n_chunk : 0;
        constexpr int n_vmem = (LOAD ? n_chunk : 0) + (VAR < 2 ? 2 : 0);
        constexpr bool NEXT_B = u < 7 || VAR < 2;
        constexpr int n_dsr = NEXT_B ? JN : 0;
        const int h = 2 * t + ph;
#pragma unroll
        for (int c = 2 * uu; c < 2 * uu + n_chunk; ++c) {
          if (WRITE) tok[((h + 2) & 3) * HALF + tpos + 256 * c] = sg[c];
          if (LOAD) sg[c] = load_chunk(h + 3, c);
        }
        u32x4(&bc)[JN] = (u & 1) ? bB : bA;
        u32x4(&bn)[JN] = (u & 1) ? bA : bB;
        if (u < 7)
          read_b(t, u + 1, bn);
        else if (NEXT_B)
          read_b(t + 1, 0, bn);
#pragma unroll
        for (int j = 0; j < JN; ++j)
#pragma unroll
          for (int i = 0; i < 2; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(wq[u][i]),
                                                                as_bf16x8(bc[j]), acc[i][j], 0, 0, 0);
        if (VAR < 2) {
#pragma unroll
          for (int i = 0; i < 2; ++i) wq[u][i] = wload((t + 1) * kPkSteps + u, i);
        }
        // Issue order inside the k-step: the staged LDS writes first (their
        // loads are four k-steps old), then the MFMAs with the next k-step's
        // fragment reads and this k-step's global loads spread between them.
        constexpr int n_mfma = 2 * JN;
        constexpr int m_dsr = n_dsr < n_mfma ? n_dsr : n_mfma;
        constexpr int m_vmem = n_vmem < n_mfma - m_dsr ? n_vmem : n_mfma - m_dsr;
        if (n_dsw > 0) __builtin_amdgcn_sched_group_barrier(0x200, n_dsw, 0);
        static_for<m_dsr>([&](auto) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        });
        static_for<m_vmem>([&](auto) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        });
        __builtin_amdgcn_sched_group_barrier(0x008, n_mfma - m_dsr - m_vmem, 0);
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
    case 2: run(std::integral_constant<int, 2>()); break;
    case 3: run(std::integral_constant<int, 3>()); break;
    case 4: run(std::integral_constant<int, 4>()); break;
    case 5: run(std::integral_constant<int, 5>()); break;
    case 6: run(std::integral_constant<int, 6>()); break;
    case 7: run(std::integral_constant<int, 7>()); break;
    default: run(std::integral_constant<int, JMAX>()); break;
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

template <bool GATED>
static hipError_t launch_packed(const moe_config& c, const void* act, const int32_t* offs,
                                const void* wp, void* out, hipStream_t st) {
  constexpr int JMAX = 8;
  const long rows = (long)c.T * c.k;
  const int N = GATED ? c.f : c.d, K = GATED ? c.d : c.f;
  const PackGeom g = pack_geom(N, K, GATED);
  const long total = (long)g.slabs * worst_row_tiles(rows, c.E, 32 * JMAX);
  const int blocks = (int)((total + 7) / 8 * 8);
  grouped_gemm_packed_kernel<GATED, JMAX><<<blocks, 256, 0, st>>>(
      static_cast<const uint16_t*>(act), offs, static_cast<const u32x4*>(wp),
      static_cast<uint16_t*>(out), c.E, N, K, (int)rows, g.slabs, 8);
  return hipGetLastError();
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
