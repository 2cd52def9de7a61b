// The expert's first GEMM (gate / up + SiLU) on FP8 operands.
//
// Pages: [SyncTax] §3.1 -- the dispatch payload crosses the all-to-all as
// per-token FP8 (one byte per element with the token's own scale and
// centre), and [V4-overlap] Waved-EP section (expert compute = L1 + Act +
// L2).  Here the first GEMM consumes those codes as they arrive, without
// decoding them to bf16 first, against expert weights quantised once to
// E4M3 with one scale per output feature:
//   x^[t, k] = c[t, k] s_t + z_t          (per-token affine payload)
//   w^[n, k] = q[n, k] s_n                (per-output-feature weights)
//   x^ . w^[n] = s_t s_n (c . q[n]) + z_t s_n sum_k q[n, k]
// so the matrix instruction multiplies raw codes (gfx950 f8f6f4 MFMA, E4M3,
// fp32 accumulation) and the epilogue applies the scales, the centre's term
// (with the per-row code sums stored next to the weights) and SiLU(a) u.
//
// FP8 gate/up image (moe_pack_weights_fp8), three 256-byte aligned parts:
//   codes [E][2F][K] uint8 -- for every group of 16 features, the 16 gate
//         rows then the 16 up rows, so that the gate and up accumulators of a
//         feature meet in the same lane (registers r and r + 8 of a 32-row
//         MFMA fragment);
//   scale [E][2F] float -- s_n = max_k |w[n, k]| / 448 (same row order);
//   csum  [E][2F] float -- sum_k of the decoded codes q[n, k] (summed
//         exactly as integers in units of 2^-9, then one float rounding).
//
// gfx950 design.  v_mfma_f32_32x32x64_f8f6f4: one 64-wide k step per MFMA;
// lane l holds row l & 31 of a 32-row fragment and k in [32 (l >> 5), +32)
// for the weights (A) and the tokens (B) alike, so the products pair up
// whatever the instruction's k order inside a lane is.  A 64-wide k stage is
// 64 bytes per row -- the same LDS geometry as the bf16 kernel of ffn.hip
// (rows of four 16-byte pieces, swizzled with (row >> 2) & 3): both operands
// reach LDS by the LDS-DMA load in a ring of stages, four waves in a 2
// (weights) x 2 (tokens) layout, the next stage's fragments read while the
// current stage's MFMAs run.  Tiles are 256 packed weight rows (128
// features) by 128 token rows, one block per tile of a worst-case grid.
// The token rows are gathered from token order through src_of (the dispatch
// writes indices only).
#include <type_traits>

#include "common.h"
#include "fp8_codec.h"
#include "tiles.h"

namespace moe {

Fp8Geom fp8_geom(const moe_config& c) {
  auto a256 = [](size_t b) { return (b + 255) & ~(size_t)255; };
  Fp8Geom g;
  g.rows = 2L * c.f;
  g.codes_bytes = (size_t)c.E * g.rows * c.d;
  g.scale_off = a256(g.codes_bytes);
  g.csum_off = g.scale_off + a256((size_t)c.E * g.rows * sizeof(float));
  g.total = g.csum_off + a256((size_t)c.E * g.rows * sizeof(float));
  return g;
}

// ------------------------------------------------------------------ packing
// One wave per packed row: the row's largest magnitude, s = max / 448
// (float32 divide), then v = w / s (float32 divide; 0 for an all-zero row),
// clamped to +-448 and encoded, and the exact sum of the decoded codes.
__global__ __launch_bounds__(256) void pack_fp8_weights_kernel(
    const uint16_t* __restrict__ wg, const uint16_t* __restrict__ wu, uint8_t* __restrict__ codes,
    float* __restrict__ scale, float* __restrict__ csum, long n_rows, int F, int K) {
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n_rows) return;  // whole wave
  const long e = row / (2L * F);
  const int r = (int)(row - e * 2L * F);
  const int feat = 16 * (r >> 5) + (r & 15);
  const u32x4* src = reinterpret_cast<const u32x4*>(((r & 31) < 16 ? wg : wu) +
                                                    ((size_t)e * F + feat) * K);
  const int nvec = K / 8;
  float m = 0.f;
  for (int v = lane; v < nvec; v += 64) {
    const u32x4 q = src[v];
    const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(wd[i])), fabsf(bf16_hi(wd[i]))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const float s = __fdiv_rn(m, kF8Max);
  double units = 0.0;  // exact: integers below 2^53
  u32x2* dst = reinterpret_cast<u32x2*>(codes + (size_t)row * K);
  for (int v = lane; v < nvec; v += 64) {
    const u32x4 q = src[v];
    const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
    uint32_t c8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float w = (i & 1) ? bf16_hi(wd[i >> 1]) : bf16_lo(wd[i >> 1]);
      float y = s > 0.f ? __fdiv_rn(w, s) : 0.f;
      y = fminf(fmaxf(y, -kF8Max), kF8Max);
      c8[i] = e4m3_encode(y);
      units += (double)e4m3_units(c8[i]);
    }
    u32x2 o;
    o.x = c8[0] | (c8[1] << 8) | (c8[2] << 16) | (c8[3] << 24);
    o.y = c8[4] | (c8[5] << 8) | (c8[6] << 16) | (c8[7] << 24);
    dst[v] = o;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) units += __shfl_xor(units, o);
  if (lane == 0) {
    scale[row] = s;
    csum[row] = __fmul_rn((float)units, 0.001953125f);  // exact: a power of two
  }
}

hipError_t launch_pack_weights_fp8(const moe_config& c, const void* wg, const void* wu,
                                   void* image, hipStream_t st) {
  const Fp8Geom g = fp8_geom(c);
  const long n_rows = (long)c.E * g.rows;
  char* base = static_cast<char*>(image);
  pack_fp8_weights_kernel<<<div_up(n_rows, 4), 256, 0, st>>>(
      static_cast<const uint16_t*>(wg), static_cast<const uint16_t*>(wu),
      reinterpret_cast<uint8_t*>(base), reinterpret_cast<float*>(base + g.scale_off),
      reinterpret_cast<float*>(base + g.csum_off), n_rows, c.f, c.d);
  return hipGetLastError();
}

// ------------------------------------------------------------------ GEMM
typedef __attribute__((address_space(3))) void f8_lds_t;
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t f8_lds_addr(const void* p) {
  return (uint32_t)(size_t)(const f8_lds_t*)p;
}
// Direct global -> LDS copy of 16 bytes per lane from sbase + voff (lane L
// writes LDS bytes [lds + 16 L, + 16); `sbase` and `lds` wave-uniform);
// inline asm so that its wait stays under this kernel's explicit vmcnt counts
// (the main loop issues no other vector-memory reads).
__device__ __forceinline__ void f8_dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(lds)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void f8_wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
// 16-byte piece q of LDS row r (rows of 64 bytes)
__device__ __forceinline__ int f8_piece(int r, int q) { return r * 4 + (q ^ ((r >> 2) & 3)); }

constexpr int kF8StageK = 64;

// WB: 32-token fragments per wave (token tile 64 WB rows).
template <int WB>
__global__ __launch_bounds__(256, (WB == 2 ? 2 : 1)) void gate_up_fp8_kernel(
    const uint8_t* __restrict__ xc, const float2* __restrict__ sz,
    const int32_t* __restrict__ src_of, int gk, int gtokens, const int32_t* __restrict__ offs,
    const uint8_t* __restrict__ wc, const float* __restrict__ wscale,
    const float* __restrict__ wcsum, uint16_t* __restrict__ h, int E, int F, int K, int rows,
    int n_tiles, int band) {
  constexpr int WA = 4;                      // weight fragments per wave
  constexpr int TW = 64 * WA;                // packed weight rows per tile (128 features)
  constexpr int TM = 64 * WB;                // token rows per tile
  constexpr int ROWS = TW + TM;              // LDS rows per stage
  constexpr int CHUNKS = ROWS * 64 / 1024;   // 1 KB DMA chunks per stage
  constexpr int DPW = CHUNKS / 4;            // DMA instructions per wave per stage
  constexpr int STAGES = WB == 2 ? 3 : 4;
  static_assert(CHUNKS % 4 == 0, "stage must split evenly over 4 waves");
  static_assert(STAGES * ROWS * 64 <= 150 * 1024, "LDS ring too large");
  __shared__ u32x4 sbuf[STAGES][ROWS * 4];
  __shared__ int s_tile[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wave == 0) place_tile<TM>(offs, E, rows, n_tiles, band, lane, s_tile);
  __syncthreads();
  const int e = s_tile[0];
  if (e < 0) return;  // block-uniform
  const int row0 = s_tile[1], row_end = s_tile[2], n_tile = s_tile[3];
  const int R2 = 2 * F;         // packed rows per expert
  const int pr0 = n_tile * TW;  // first packed row of the tile
  const int nk = K / kF8StageK;

  // ---- DMA assignment: wave w copies chunks w + 4 i of every stage; chunk c
  // holds LDS rows 16 c .. 16 c + 15 (weight rows first); lane l lands at row
  // 16 c + l / 4, physical piece l % 4, fetching logical piece
  // (l & 3) ^ ((row >> 2) & 3) = (l & 3) ^ ((l >> 4) & 3).
  // Byte offsets (32-bit: one expert's codes and T rows of codes stay below
  // 2^31 bytes) from the expert's weight codes or from the token codes.
  const int lq = (lane & 3) ^ ((lane >> 4) & 3);
  const uint8_t* wbase = wc + (size_t)e * R2 * K;
  uint32_t goff[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int r = 16 * (wave + 4 * i) + (lane >> 2);  // chunk wave + 4 i is uniform per i
    if (r < TW) {
      const int pr = min(pr0 + r, R2 - 1);  // rows past the last feature feed unstored outputs
      goff[i] = (uint32_t)pr * (uint32_t)K + lq * 16u;
    } else {
      const int p = min(row0 + (r - TW), row_end - 1);
      const int t = min(max(src_of[p] / gk, 0), gtokens - 1);
      goff[i] = (uint32_t)t * (uint32_t)K + lq * 16u;
    }
  }

  // ---- fragments: wave (wn, wm) owns weight rows wn 128 .. + 127 (fragments
  // of 32) and token rows wm 32 WB .. (fragments of 32)
  const int wn = wave >> 1, wm = wave & 1;
  const int lk = lane >> 5;
  const int arow0 = wn * 32 * WA + (lane & 31);
  const int tok0 = wm * 32 * WB;
  const int jn =
      __builtin_amdgcn_readfirstlane(min(WB, max(0, (row_end - row0 - tok0 + 31) >> 5)));
  const int brow0 = TW + tok0 + (lane & 31);

  f32x16 acc[WA][WB];
#pragma unroll
  for (int i = 0; i < WA; ++i)
#pragma unroll
    for (int j = 0; j < WB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const uint32_t lds0 = f8_lds_addr(&sbuf[0][0]);
  auto issue = [&](int kt) {
    const uint32_t sbase = lds0 + (uint32_t)(kt % STAGES) * (ROWS * 64u);
    const uint8_t* wk = wbase + (size_t)kt * kF8StageK;
    const uint8_t* xk = xc + (size_t)kt * kF8StageK;
#pragma unroll
    for (int i = 0; i < DPW; ++i)  // chunks below TW / 16 are weight rows (wave-uniform)
      f8_dma16(16 * (wave + 4 * i) < TW ? wk : xk, goff[i],
               sbase + (uint32_t)(wave + 4 * i) * 1024u);
  };
  auto main_loop = [&](auto jn_c) {
    constexpr int JN = decltype(jn_c)::value;
    struct Frags {
      i32x8 a[WA];
      i32x8 b[WB];
    };
    auto frag = [&](const u32x4* sb, int row) -> i32x8 {
      const u32x4 p0 = sb[f8_piece(row, 2 * lk)], p1 = sb[f8_piece(row, 2 * lk + 1)];
      const i32x8 v = {(int)p0.x, (int)p0.y, (int)p0.z, (int)p0.w,
                       (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w};
      return v;
    };
    auto load_frags = [&](int kt, Frags& Fr) {
      const u32x4* sb = sbuf[kt % STAGES];
#pragma unroll
      for (int i = 0; i < WA; ++i) Fr.a[i] = frag(sb, arow0 + 32 * i);
#pragma unroll
      for (int j = 0; j < JN; ++j) Fr.b[j] = frag(sb, brow0 + 32 * j);
    };
    auto mfma_stage = [&](const Frags& Fr) {
#pragma unroll
      for (int j = 0; j < JN; ++j)
#pragma unroll
        for (int i = 0; i < WA; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(Fr.a[i], Fr.b[j], acc[i][j],
                                                                      0, 0, 0, 0, 0, 0);
    };
    // Stage j goes to LDS buffer j % STAGES.  Stage kt's fragments are read
    // during step kt - 1.  End of step kt: wait for this wave's copies of
    // stage kt + 2, barrier (all copies of kt + 2 visible; nobody reads
    // stages kt, kt + 1 any more), then refill buffer kt % STAGES with stage
    // kt + STAGES.
    // wait until this wave's copies of every stage before `later` younger
    // ones are in (vmcnt takes an immediate)
    auto wait_later = [&](int later) {
      switch (later) {
        case 0: f8_wait_vm_barrier<0>(); break;
        case 1: f8_wait_vm_barrier<DPW>(); break;
        case 2: f8_wait_vm_barrier<2 * DPW>(); break;
        case 3: f8_wait_vm_barrier<3 * DPW>(); break;
        default: f8_wait_vm_barrier<4 * DPW>(); break;
      }
    };
    static_assert(STAGES <= 6, "wait_later covers up to four younger stages");
    auto wait_for = [&](int j) { wait_later(min(nk - 1, j + STAGES - 3) - j); };
#pragma unroll
    for (int i = 0; i < STAGES; ++i)
      if (i < nk) issue(i);
    wait_later(max(0, min(nk - 1, STAGES - 1) - 1));  // stages 0 and 1 visible
    Frags F0, F1;
    if (JN > 0) load_frags(0, F0);
    auto step = [&](int kt, Frags& cur, Frags& nxt) {
      if (JN > 0) {
        load_frags(min(kt + 1, nk - 1), nxt);  // the last step re-reads the final stage
        mfma_stage(cur);
      }
      if (kt + 2 < nk)
        wait_for(kt + 2);
      else
        f8_wait_vm_barrier<0>();
      if (kt + STAGES < nk) issue(kt + STAGES);
    };
    for (int kt = 0; kt < nk; kt += 2) {  // nk is even (K is a multiple of 128)
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
  // [token fragment j, lane & 31].  Rows 0..15 of a fragment are the gate
  // rows and rows 16..31 the up rows of the same 16 features, so registers
  // 4 g + r (g < 2) and 4 g + 8 + r hold gate and up of one feature.
  const float* sc = wscale + (size_t)e * R2;
  const float* cs = wcsum + (size_t)e * R2;
#pragma unroll
  for (int j = 0; j < WB; ++j) {
    const int p = row0 + tok0 + 32 * j + (lane & 31);
    if (j >= jn || p >= row_end) continue;
    const int t = min(max(src_of[p] / gk, 0), gtokens - 1);
    const float2 tz = sz[t];  // (s_t, z_t)
#pragma unroll
    for (int i = 0; i < WA; ++i) {
      const int prf = pr0 + wn * 32 * WA + 32 * i;  // first packed row of the fragment
      if (prf >= R2) continue;
      const int fb = prf / 2;                       // its first feature (16 per 32 rows)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int rg = prf + 8 * g + 4 * lk;        // gate rows rg .. rg + 3, up rows + 16
        const float4 sg = *reinterpret_cast<const float4*>(sc + rg);
        const float4 cg = *reinterpret_cast<const float4*>(cs + rg);
        const float4 su = *reinterpret_cast<const float4*>(sc + rg + 16);
        const float4 cu = *reinterpret_cast<const float4*>(cs + rg + 16);
        const float sgv[4] = {sg.x, sg.y, sg.z, sg.w}, cgv[4] = {cg.x, cg.y, cg.z, cg.w};
        const float suv[4] = {su.x, su.y, su.z, su.w}, cuv[4] = {cu.x, cu.y, cu.z, cu.w};
        float hv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = tz.x * sgv[r] * acc[i][j][4 * g + r] + tz.y * sgv[r] * cgv[r];
          const float u = tz.x * suv[r] * acc[i][j][4 * g + 8 + r] + tz.y * suv[r] * cuv[r];
          hv[r] = a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)) * u;
        }
        u32x2 pk;
        pk.x = pack_bf16x2(hv[0], hv[1]);
        pk.y = pack_bf16x2(hv[2], hv[3]);
        *reinterpret_cast<u32x2*>(h + (size_t)p * F + fb + 8 * g + 4 * lk) = pk;
      }
    }
  }
}

// Tile shape: 256 weight rows x 128 tokens, two blocks per CU, so that one
// block's MFMAs run while the other waits for its stages.  Measured against
// 256-token tiles (one block per CU, four stages) and against 128-token tiles
// with one block per CU and four or six stages: T8192-E256 2.71 ms against
// 2.98 / 3.25 / 3.23 ms, T1024-E8 289 against 362 / 375 / 373 us.
hipError_t launch_ffn_gate_up_fp8_gather(const moe_config& c, const void* x_codes,
                                         const float* scale_zero, const int32_t* src_of,
                                         const int32_t* offs, const void* image, void* h,
                                         hipStream_t st) {
  const Fp8Geom g = fp8_geom(c);
  const long rows = (long)c.T * c.k;
  const int n_tiles = div_up(g.rows, 256);
  constexpr int wb = 2;
  const long total = (long)n_tiles * worst_row_tiles(rows, c.E, 64 * wb);
  const int blocks = (int)((total + 7) / 8 * 8);
  const char* base = static_cast<const char*>(image);
  const auto* xc = static_cast<const uint8_t*>(x_codes);
  const auto* szp = reinterpret_cast<const float2*>(scale_zero);
  const auto* wc = reinterpret_cast<const uint8_t*>(base);
  const auto* ws = reinterpret_cast<const float*>(base + g.scale_off);
  const auto* wcs = reinterpret_cast<const float*>(base + g.csum_off);
  auto* hp = static_cast<uint16_t*>(h);
  gate_up_fp8_kernel<wb><<<blocks, 256, 0, st>>>(xc, szp, src_of, c.k, c.T, offs, wc, ws, wcs, hp,
                                                 c.E, c.f, c.d, (int)rows, n_tiles, 8);
  return hipGetLastError();
}

}  // namespace moe
