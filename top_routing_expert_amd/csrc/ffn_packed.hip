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
// once while the tokens stay in L2.  Packed once (at load time) into MFMA
// fragment order, the weights go straight from HBM into the registers of the
// one wave that uses them: each wave instruction reads 1 KB of consecutive
// bytes.  Only the tokens, shared by all four waves, pass through LDS.
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
// Kernel (persistent, one block of 4 waves per CU):
//  * Tile shapes: a whole slab (wave w: weight fragments (w, 0..1), 256
//    accumulators) x up to 256 token rows of one expert; or, when whole-slab
//    tiles cannot fill the chip twice over, half a slab (wave w: fragment
//    (w, half)) x up to 320 rows.  Half-slab tiles of more than 160 rows run
//    the waves as a 2 x 2 grid (two weight fragments x half the token
//    fragments each), so every token fragment read from LDS feeds two MFMAs.
//    An expert's rows are split evenly over its row tiles, so the tiles of
//    one slab run side by side and share the weight stream through L2.
//  * k loop in iterations of 128 (8 MFMA k-steps).  Weight fragments of
//    k-step s+8 are loaded into the register slot of k-step s right after the
//    MFMAs that use it.  Token rows are copied straight from global memory
//    into a ring of 64-wide k half-stages in LDS (four slots, three for
//    320-row tiles), D = slots - 1 half-stages ahead; LDS rows of 128 bytes,
//    16-byte pieces XOR-swizzled with (row >> 1) & 7 so the 16 lanes of a
//    16-byte read hit 16 bank groups.  One barrier per half-stage.
//  * Both streams share the in-order load counter, so the kernel issues its
//    loads itself in a fixed order (PkSched) and waits with exact counts: a
//    wait for a token half-stage never drains weight loads issued for later
//    k-steps, and vice versa.
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
constexpr int kCopySteps = 4;  // k-steps of a half-stage over which its copies are spread
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

// The same plain (non-gated) image of a matrix W'[e][n][k] that is stored
// transposed: W'[e][n][k] = src0[e][k][n] for k < K0, src1[e][k - K0][n] above
// (src0 [E, K0, F], src1 [E, K - K0, F]).  The backward's activation-gradient
// products use it: W_d^T (F = f, K = d) and [W_g; W_u]^T (F = d, K = 2 f).
// A load-time layout like the forward's; the reads are strided.
__global__ void pack_weights_t_kernel(const uint16_t* __restrict__ src0,
                                      const uint16_t* __restrict__ src1, u32x4* __restrict__ dst,
                                      int F, int K0, int K, int slabs, int kp, size_t total) {
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
    const int feat = slab * 256 + w * 64 + i * 32 + (lane & 31);
    const int k = ks * 16 + 8 * (lane >> 5);
    uint16_t v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int kk = k + q;
      v[q] = 0;
      if (feat < F && kk < K)
        v[q] = kk < K0 ? src0[(e * K0 + kk) * (size_t)F + feat]
                       : src1[(e * (K - K0) + (kk - K0)) * (size_t)F + feat];
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = (uint32_t)v[2 * q] | ((uint32_t)v[2 * q + 1] << 16);
    dst[p] = o;
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

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource (gfx950) over `bytes` bytes at `base`; every word is
// made wave-uniform so the descriptor lives in scalar registers.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));  // stride 0
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = kBufferFlags;
  return r;
}

// The main loop issues its loads itself and waits for them with explicit
// counts: the weight loads (into registers) and the token copies (straight
// into LDS) share one in-order counter, and a compiler-placed wait for one
// would also drain the other's far-ahead loads.
//
// 16 bytes per lane of a weight stream into registers (buffer_load_dwordx4).
template <int IMM>
__device__ __forceinline__ u32x4 wload_async(i32x4 rsrc, uint32_t voff, int soff) {
  u32x4 v;
  asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen offset:%4"
               : "=v"(v)
               : "v"(voff), "s"(rsrc), "s"(soff), "n"(IMM));
  return v;
}
// Direct global -> LDS copy: lane L writes LDS bytes [lds + 16 L, lds + 16 L + 16)
// from sbase + voff (wave-uniform `sbase` and `lds`).
__device__ __forceinline__ void dma_async(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(lds)
               : "memory", "m0");
}
// Wait until at most N loads are in flight; the weight registers are passed
// through so that no use of them can be placed before the wait.
template <int N>
__device__ __forceinline__ void wait_vm(u32x4& a) {
  asm volatile("s_waitcnt vmcnt(%1)" : "+v"(a) : "n"(N));
}
template <int N>
__device__ __forceinline__ void wait_vm(u32x4& a, u32x4& b) {
  asm volatile("s_waitcnt vmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
// Wait until at most N loads are in flight and this wave's LDS reads are
// done, then barrier: afterwards every wave's copies issued before the last
// N loads are in LDS, and no wave still reads a slot about to be refilled.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Wait until at most N loads are in flight, then barrier, leaving this wave's
// LDS reads in flight: for a barrier after which only slots that no read in
// flight targets are refilled.
template <int N>
__device__ __forceinline__ void wait_vm_barrier_reads_in_flight() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Load schedule of the main loop (compile-time).  k-step s = 8 t + u of
// iteration t, half-stage h = 2 t + (u >> 2), uu = u & 3.  Every k-step of a
// FULL iteration starts with its wait for weight k-step s and then issues,
// spread over its MFMAs so that the four waves never queue a burst of loads
// at the texture unit at once: the token copies of chunks [cl(uu), cl(uu+1))
// of half-stage h + D (the first na(uu) of them, "A", and the rest, "B") and
// WL weight loads of k-step s + 8, in the order A, w0, B, w1 (WL = 2) or A,
// B, w0 (WL = 1).  The last iteration issues nothing.  The prologue issues
// the copies of half-stages 0..D-3 and then a pseudo iteration -1 in the FULL
// order, so the counts below hold from the first k-step on.  Loads past the
// end of the tile read clamped (real) addresses and land in slots nobody
// reads.  A half-stage's copies go out over its first KC k-steps.  The
// loads share one in-order counter, so a wait for a half-stage's copies also
// waits for every weight load issued before its last copy.
struct PkSched {
  int JN, WL, D, KC;  // KC: k-steps of a half-stage that issue its copies (1, 2 or 4)
  constexpr int cl(int uu) const { return JN * (uu < KC ? uu : KC) / KC; }  // first chunk of k-step uu
  constexpr int nc(int uu) const { return cl(uu + 1) - cl(uu); }
  constexpr int na(int uu) const { return (nc(uu) + 1) / 2; }
  constexpr int nb(int uu) const { return nc(uu) - na(uu); }
  // loads issued in k-step uu after its last copy
  constexpr int tail(int uu) const { return WL == 2 && nb(uu) == 0 ? 2 : 1; }
  // the k-step of a half-stage that issues its last copy
  constexpr int lastk() const {
    int k = 0;
    for (int q = 0; q < 4; ++q)
      if (nc(q) > 0) k = q;
    return k;
  }
  // loads issued after the last copy of a half-stage, to the end of that half-stage
  constexpr int rest() const { return tail(lastk()) + (3 - lastk()) * WL; }
  // loads issued after weight k-step s (the last load of k-step s - 8) up to
  // the wait at the start of k-step s: k-steps s-7 .. s-1, s in a FULL iteration
  constexpr int w_full(int u) const { return 7 * WL + 2 * JN - nc(u & 3); }
  // the same in the last iteration (no loads of its own), k-step u of it
  constexpr int w_last(int u) const {
    int n = 0;
    for (int k = u + 1; k < 8; ++k) n += nc(k & 3) + WL;
    return n;
  }
  // D = 2: at the end of half-stage h, loads issued after the last copy of
  // half-stage h + 1 (issued during half-stage h - 1): the rest of that
  // half-stage and half-stage h -- or, in the first half of the last
  // iteration, nothing more; before the first barrier, after half-stage 0's
  // last copy
  constexpr int x_full() const { return rest() + (D - 1) * (JN + 4 * WL); }
  constexpr int x_last() const { return rest() + (D - 2) * (JN + 4 * WL); }
  constexpr int x_first() const { return rest() + JN + 4 * WL; }
  // D >= 3 (early publication): the end of half-stage h waits for the copies
  // of h + 2, so that the B fragments of h + 1's first k-step can be read
  // before that barrier; they were issued during half-stage h + 2 - D.
  // Before the first barrier: after half-stage 1's last copy (pseudo
  // iteration, first half, for D = 3; the prologue for D = 4).
  constexpr int x_full_early() const { return rest() + (D - 2) * (JN + 4 * WL); }
  constexpr int x_first_early() const {
    return D == 3 ? rest() + JN + 4 * WL : (D - 2) * JN + 8 * WL;
  }
};

// Specialisation of a tile of J live token fragments: the fragment count
// (at most JMAX) and whether its waves run as 2 x 2 pairs (half-slab tiles of
// more than JMAX / 2 fragments).
template <int J, int JMAX, int WF>
struct JnSel {
  static constexpr int jn = J < JMAX ? J : JMAX;
  using N = std::integral_constant<int, jn>;
  using P = std::integral_constant<bool, (WF == 1 && 2 * jn > JMAX)>;
};

// JMAX: 32-token fragments per tile (tile = 32 JMAX tokens); WF: 32-row
// weight fragments per wave (2: a tile spans a whole slab; 1: half a slab, for
// GEMMs with too few tiles to fill the chip).
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
//
// GATHER: the activation rows are gathered from token order: tile row p reads
// act row src_of[p] / gk (clamped into [0, gtokens)), so the permuted copy of
// the activations is never written.
// SAVE (gated only): also write the pre-activations a and u next to h.
template <bool GATED, int JMAX, int WF, bool GATHER, bool SAVE = false>
__global__ __launch_bounds__(256, 1) void grouped_gemm_packed_kernel(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ offs,
    const u32x4* __restrict__ wp, uint16_t* __restrict__ out, int E, int N, int K, int rows,
    int slabs, int band, bool sized, const int32_t* __restrict__ src_of, int gk, int gtokens,
    uint16_t* __restrict__ save_a, uint16_t* __restrict__ save_u) {
  constexpr int TM = 32 * JMAX;
  constexpr int TN = GATED ? 128 : 256;       // output features per slab
  constexpr int HB = TM * 128;                // bytes of one 64-wide k half-stage
  constexpr int NSLOT = 4 * HB <= 150 * 1024 ? 4 : 3;  // LDS ring of half-stages
  constexpr int D = NSLOT - 1;                // half-stages of copy lookahead
  constexpr int NT = WF == 2 ? 1 : 2;         // tiles per slab
  static_assert(JMAX <= 10 && (WF == 1 || WF == 2), "tile shape");
  __shared__ __attribute__((aligned(16))) unsigned char tokb[NSLOT * HB];
  __shared__ int s_tile[4];
  __shared__ int s_total;
  // expert order: every expert's rows and first tile, built once (wave 0)
  __shared__ int s_o0[kTileTableMax], s_o1[kTileTableMax], s_start[kTileTableMax];

  const int G = (int)gridDim.x;
  const int qp = (G >> 3) * (int)(blockIdx.x & 7) + (int)(blockIdx.x >> 3);
  if (threadIdx.x < 64) {
    const int n = sized ? count_row_tiles<TM>(offs, E, rows, (int)threadIdx.x) * slabs * NT
                        : build_tile_table<TM>(offs, E, rows, slabs * NT, (int)threadIdx.x, s_o0,
                                               s_o1, s_start);
    if (threadIdx.x == 0) s_total = n;
  }
  const uint32_t lds0 = (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)tokb;
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
    if (L < s_total) {
      if (sized)
        locate_tile<TM>(offs, E, rows, slabs * NT, band, L, lane, s_tile, true);
      else
        locate_in_table<TM>(s_o0, s_o1, s_start, E, slabs * NT, band, L, lane, s_tile);
    }
  }
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(s_tile[0]);
  if (e < 0) break;  // block-uniform; later rounds only hold larger tile numbers
  const int row0 = __builtin_amdgcn_readfirstlane(s_tile[1]);
  const int row_end = __builtin_amdgcn_readfirstlane(s_tile[2]);
  const int wt = __builtin_amdgcn_readfirstlane(s_tile[3]);
  const int slab = wt / NT, half = wt % NT;
  const int nrow = min(row_end - row0, TM);
  const int jn = (nrow + 31) >> 5;  // live token fragments, 1..JMAX
  const int kp = (K + kPkIterK - 1) / kPkIterK * kPkIterK;
  const int nit = kp / kPkIterK;
  const int hlast = K / 64 - 1;  // half-stages past K re-read the last real one (zero weights)

  const uint32_t wl = (uint32_t)lane * 16u;
  const uint32_t sbytes = (uint32_t)(kp / 16) * 2048u;  // one packed weight stream

  // Token copies.  Half-stage h = k range [64 h, 64 h + 64) of the tile's rows,
  // in LDS slot h % NSLOT: rows of 128 bytes, the 16-byte piece q of row r at
  // q ^ ((r >> 1) & 7), so the 16 lanes served together by a 16-byte LDS read
  // (16 consecutive rows, one piece) hit 16 different bank groups.  Chunk c =
  // tile rows 32c..32c+31; this wave copies rows 32c + 8 wave .. + 7 with one
  // instruction: lane l fills LDS row 32c + 8 wave + l/8, piece l & 7, with
  // the logical piece (l & 7) ^ swizzle of that row.  Only the last chunk can
  // reach past the expert's rows; it copies a clamped (real) row instead.
  const int trow = 8 * wave + (lane >> 3);
  const int lp = (lane & 7) ^ ((trow >> 1) & 7);
  const char* abase = reinterpret_cast<const char*>(act);
  // fragment reads: token row 32 j + (lane & 31), piece (2 uu + lk) ^ ((row >> 1) & 7)
  const int lk = lane >> 5, bsw = (lane >> 1) & 7;
  const uint32_t rd0 = (uint32_t)(lane & 31) * 128u;

  // PAIR (half-slab tiles of more than JMAX / 2 fragments): the waves form a
  // 2 x 2 grid, wave 2a + b computing the slab's fragments `half` of packed
  // streams 2a and 2a + 1 on token fragments [b JW, b JW + JW), so that every
  // token fragment read from LDS feeds two MFMAs.  Otherwise wave w computes
  // its own stream's fragments (both, or `half`) on every token fragment.
  auto run = [&](auto jn_c, auto pair_c) {
    constexpr int JN = decltype(jn_c)::value;
    constexpr bool PAIR = decltype(pair_c)::value;
    constexpr int WL = PAIR ? 2 : WF;              // weight fragments of this wave
    constexpr int JW = PAIR ? (JN + 1) / 2 : JN;  // token fragments of this wave
    const int jb = PAIR ? (wave & 1) * JW : 0;
    // With JN odd the second pair's last fragment (JN) lies past the tile's
    // rows; it reads stale LDS rows of the slot and is never stored.
    const int pw = PAIR ? (wave & ~1) : wave;      // first packed stream of this wave
    static_assert(!PAIR || JN % 2 == 0 || JN < JMAX, "fragment JN must lie inside the slot");
    static_assert(D >= 2 && D <= 4, "ring depth");
    constexpr PkSched S{JN, WL, D, kCopySteps};
    // The wave's weight stream(s) as one buffer resource: fragment i of
    // k-step s of stream pw + q at q * sbytes + s * 2048 + i * 1024.
    const i32x4 wrsrc =
        make_rsrc(wp + (((size_t)e * slabs + slab) * 4 + pw) * ((size_t)(kp / 16) * 128),
                  (PAIR ? 2u : 1u) * sbytes);
    const uint32_t wl1 = wl + (PAIR ? sbytes : 0u);
    const int wfrag0 = WF == 2 ? 0 : half * 1024;
    // Plain rows: the tile's first row goes into the 64-bit scalar base and
    // the per-lane offsets stay inside the tile (< TM rows of K elements), so
    // they fit 32 bits for any K (the backward's k = 2 f included).
    const char* tbase = GATHER ? abase : abase + (size_t)row0 * K * 2;
    const uint32_t toff0 = ((uint32_t)trow * (uint32_t)K + 8u * lp) * 2u;
    const uint32_t tofl =
        ((uint32_t)min(32 * (JN - 1) + trow, nrow - 1) * (uint32_t)K + 8u * lp) * 2u;
    const size_t cstride = (size_t)64 * K;  // bytes of 32 rows
    // GATHER: byte offset of this lane's source row for every chunk
    uint32_t goff[GATHER ? JN : 1];
    if constexpr (GATHER) {
#pragma unroll
      for (int c = 0; c < JN; ++c) {
        const int p = row0 + min(32 * c + trow, nrow - 1);
        const int t = min(max(src_of[p] / gk, 0), gtokens - 1);
        goff[c] = ((uint32_t)t * (uint32_t)K + 8u * lp) * 2u;
      }
      // The compiler waits for its own loads with counts that do not know of
      // the asm loads below: every offset is final before the first of them.
#pragma unroll
      for (int c = 0; c < JN; ++c) asm volatile("" : "+v"(goff[c]));
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    auto copy_chunk = [&](int h, int c) {
      const char* hb = tbase + (size_t)min(h, hlast) * 128;
      const uint32_t lds = lds0 + (uint32_t)((h % NSLOT) * HB + (32 * c + 8 * wave) * 128);
      if constexpr (GATHER)
        dma_async(hb, goff[c], lds);
      else if (c == JN - 1)
        dma_async(hb, tofl, lds);
      else
        dma_async(hb + c * cstride, toff0, lds);
    };
    // weight k-step s (clamped into the stream: loads past the end are re-reads)
    const int slast = kp / 16 - 1;
    auto wload = [&](int s, auto i_c) -> u32x4 {
      constexpr int I = decltype(i_c)::value;
      if constexpr (PAIR)
        return wload_async<0>(wrsrc, I ? wl1 : wl, min(s, slast) * 2048 + wfrag0);
      else
        return wload_async<I * 1024>(wrsrc, wl, min(s, slast) * 2048 + wfrag0);
    };
    auto rdb = [&](int h, int uu, int j) -> u32x4 {
      const int q = (2 * uu + lk) ^ bsw;
      return *reinterpret_cast<const u32x4*>(tokb + (h % NSLOT) * HB + j * 4096 + rd0 + q * 16);
    };

    u32x4 wq[8][WL];
    u32x4 bq[JW];
    // prologue: copies of half-stages 0..D-3, then pseudo iteration -1
    for (int h = 0; h < D - 2; ++h)
      static_for<JN>([&](auto c) { copy_chunk(h, c); });
    static_for<8>([&](auto u_c) {
      constexpr int u = decltype(u_c)::value, uu = u & 3;
      // the order of a FULL k-step: A, w0, B, w1 or A, B, w0
      static_for<S.na(uu)>([&](auto cc) { copy_chunk(D - 2 + (u >> 2), S.cl(uu) + cc); });
      if constexpr (WL == 2) wq[u][0] = wload(u, std::integral_constant<int, 0>());
      static_for<S.nb(uu)>([&](auto cc) { copy_chunk(D - 2 + (u >> 2), S.cl(uu) + S.na(uu) + cc); });
      wq[u][WL - 1] = wload(u, std::integral_constant<int, WL - 1>());
    });
    // With D = 3 every half-stage is published one half-stage before it is
    // read (so the B fragments of a half-stage's first k-step can be read
    // during the last k-step of the one before); with the three-slot ring
    // (D = 2) the copies of h + 1 can only be awaited at the end of h.
    constexpr bool EARLY = D >= 3;
    if constexpr (EARLY)
      wait_vm_barrier<S.x_first_early()>();
    else
      wait_vm_barrier<S.x_first()>();
    static_for<JW>([&](auto j) { bq[j] = rdb(0, 0, jb + j); });
    // the accumulators come to life only now
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc[WL][JW];
#pragma unroll
    for (int i = 0; i < WL; ++i)
#pragma unroll
      for (int j = 0; j < JW; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // LAST = 0: full iteration; 1: the last one (issues no loads)
    auto iter = [&](int t, auto last_c) {
      constexpr bool LAST = decltype(last_c)::value;
      __builtin_amdgcn_sched_barrier(0);
      static_for<8>([&](auto u_c) {
        constexpr int u = decltype(u_c)::value;
        constexpr int ph = u >> 2, uu = u & 3;
        const int h = 2 * t + ph;
        if constexpr (WL == 2) {
          wait_vm<LAST ? S.w_last(u) : S.w_full(u)>(wq[u][0], wq[u][1]);
        } else {
          wait_vm<LAST ? S.w_last(u) : S.w_full(u)>(wq[u][0]);
        }
        // The next k-step's B fragments are read during this k-step's MFMAs
        // (EARLY), or -- D = 2 -- for the first k-step of the next half-stage
        // after the barrier that publishes its copies.
        constexpr bool NEXT_B = EARLY ? !(LAST && u == 7) : uu != 3;
        const int hn = uu == 3 ? h + 1 : h;
        constexpr int un = (uu + 1) & 3;
        // MFMAs of weight fragment I on token fragments [J0, J1), each B
        // fragment read again right after its last MFMA of the k-step
        auto mf = [&](auto i_c, auto j0_c, auto j1_c) {
          constexpr int I = decltype(i_c)::value, J0 = decltype(j0_c)::value;
          constexpr int J1 = decltype(j1_c)::value;
          constexpr bool RD = NEXT_B && I == WL - 1;
          static_for<J1 - J0>([&](auto jj) {
            constexpr int j = J0 + decltype(jj)::value;
            acc[I][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(wq[u][I]),
                                                                as_bf16x8(bq[j]), acc[I][j], 0, 0, 0);
            if constexpr (RD) bq[j] = rdb(hn, un, jb + j);
          });
          static_for<J1 - J0>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if constexpr (RD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          });
          __builtin_amdgcn_sched_barrier(0);
        };
        // token copies of chunks [C0, C0 + NCP) of half-stage h + D
        auto copies = [&](auto c0_c, auto n_c) {
          if constexpr (!LAST) {
            static_for<decltype(n_c)::value>(
                [&](auto cc) { copy_chunk(h + D, decltype(c0_c)::value + cc); });
            __builtin_amdgcn_sched_barrier(0);
          }
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using CA = std::integral_constant<int, S.cl(uu)>;
        using NA = std::integral_constant<int, S.na(uu)>;
        using CB = std::integral_constant<int, S.cl(uu) + S.na(uu)>;
        using NB = std::integral_constant<int, S.nb(uu)>;
        using JE = std::integral_constant<int, JW>;
        if constexpr (WL == 2) {
          // i-major: weight fragment 0 is free after the first JW MFMAs,
          // fragment 1 after the last; the copies sit halfway through each half
          using PA = std::integral_constant<int, (JW / 2 > 1 ? JW / 2 : 1)>;
          mf(I0(), I0(), PA());
          copies(CA(), NA());
          mf(I0(), PA(), JE());
          if constexpr (!LAST) wq[u][0] = wload(8 * t + u + 8, I0());
          __builtin_amdgcn_sched_barrier(0);
          mf(I1(), I0(), PA());
          copies(CB(), NB());
          mf(I1(), PA(), JE());
          if constexpr (!LAST) wq[u][1] = wload(8 * t + u + 8, I1());
        } else {
          using PA = std::integral_constant<int, (JW / 3 > 1 ? JW / 3 : 1)>;
          using PB = std::integral_constant<int, (2 * JW / 3 > PA::value ? 2 * JW / 3 : PA::value)>;
          mf(I0(), I0(), PA());
          copies(CA(), NA());
          mf(I0(), PA(), PB());
          copies(CB(), NB());
          mf(I0(), PB(), JE());
          if constexpr (!LAST) wq[u][0] = wload(8 * t + u + 8, I0());
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (EARLY) {
          // publish half-stage h + 2 (the last iteration has nothing left to
          // publish).  The reads in flight here are of half-stage h + 1; the
          // copies issued after this barrier refill slot h, whose reads were
          // all consumed by this half-stage's MFMAs.
          if constexpr (uu == 3 && !LAST) {
            wait_vm_barrier_reads_in_flight<S.x_full_early()>();
            __builtin_amdgcn_sched_barrier(0);
          }
        } else if constexpr (uu == 3 && !(LAST && ph == 1)) {
          if constexpr (!LAST)
            wait_vm_barrier<S.x_full()>();
          else
            wait_vm_barrier<S.x_last()>();
          static_for<JW>([&](auto j) { bq[j] = rdb(h + 1, 0, jb + j); });
          __builtin_amdgcn_sched_barrier(0);
        }
      });
    };
    int t = 0;
    for (; t + 1 < nit; ++t) iter(t, std::false_type());
    iter(t, std::true_type());
    // copies issued past the end are still in flight: drain them before the
    // next tile reuses the ring
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // epilogue: acc[ii][jj][4 g + r] = C[fragment row 8 g + 4 lk + r][token lane & 31]
    if constexpr (WF == 2 && !SAVE) {
      // Whole-slab tiles: the bf16 output tile goes through the (now idle)
      // LDS ring, rows of TN features, 16-byte pieces XOR-swizzled with the
      // row so that a store's 32 rows land on different banks, then out in
      // whole row segments: every store instruction writes 64 / PPR full
      // rows of the tile instead of 16 bytes in each of 32 rows.
      constexpr int RB = TN * 2;    // bytes of one row of the output tile
      constexpr int PPR = RB / 16;  // 16-byte pieces per row
      constexpr int RPI = 64 / PPR; // rows per store instruction
      static_assert(TM * RB <= NSLOT * HB, "the output tile must fit the ring");
      __syncthreads();  // every wave's last fragment reads of the ring are done
      auto put = [&](int r, int nl, u32x2 v) {  // tile row r, tile feature nl (a multiple of 4)
        const int q = nl >> 3;
        *reinterpret_cast<u32x2*>(tokb + r * RB + ((q ^ (r & (PPR - 1))) << 4) +
                                  ((nl >> 2) & 1) * 8) = v;
      };
#pragma unroll
      for (int jj = 0; jj < JW; ++jj) {
        const int r = 32 * jj + (lane & 31);
#pragma unroll
        for (int ii = 0; ii < WL; ++ii) {
          if (GATED) {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
              float hv[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float gt = acc[ii][jj][4 * g + q], up = acc[ii][jj][4 * g + 8 + q];
                hv[q] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
              }
              u32x2 pk;
              pk.x = pack_bf16x2(hv[0], hv[1]);
              pk.y = pack_bf16x2(hv[2], hv[3]);
              put(r, wave * (TN / 4) + 16 * ii + 8 * g + 4 * lk, pk);
            }
          } else {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              u32x2 pk;
              pk.x = pack_bf16x2(acc[ii][jj][4 * g], acc[ii][jj][4 * g + 1]);
              pk.y = pack_bf16x2(acc[ii][jj][4 * g + 2], acc[ii][jj][4 * g + 3]);
              put(r, wave * (TN / 4) + 32 * ii + 8 * g + 4 * lk, pk);
            }
          }
        }
      }
      __syncthreads();
      const int q = lane % PPR;
      const int n = slab * TN + 8 * q;
      // Pass i of this wave covers tile rows wave RPI + 4 RPI i + [0, RPI): every
      // row read lies inside the staged tile.  Eight reads go out before their
      // stores (a read-wait-store loop waited for every LDS read in turn).
      constexpr int STEP = 4 * RPI, PASSES = 32 * JW / STEP, BATCH = 8;
      static_assert(32 * JW % STEP == 0, "whole passes");
#pragma unroll
      for (int i0 = 0; i0 < PASSES; i0 += BATCH) {
        u32x4 v[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
          const int r = wave * RPI + (i0 + i) * STEP + lane / PPR;
          if (i0 + i < PASSES)
            v[i] = *reinterpret_cast<const u32x4*>(tokb + r * RB + ((q ^ (r & (PPR - 1))) << 4));
        }
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
          const int r = wave * RPI + (i0 + i) * STEP + lane / PPR;
          if (i0 + i < PASSES && r < nrow && n < N)
            *reinterpret_cast<u32x4*>(out + (size_t)(row0 + r) * N + n) = v[i];
        }
      }
      return;
    }
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      const int p = row0 + 32 * (jb + jj) + (lane & 31);
      if (p >= row_end) continue;
      uint16_t* orow = out + (size_t)p * N;
#pragma unroll
      for (int ii = 0; ii < WL; ++ii) {
        const int i = WF == 2 ? ii : half;  // weight fragment of the stream
        const int nb = slab * TN + (PAIR ? pw + ii : wave) * (TN / 4);
        if (GATED) {
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const int n = nb + 16 * i + 8 * g + 4 * lk;
            if (n >= N) continue;
            float hv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float gt = acc[ii][jj][4 * g + r], up = acc[ii][jj][4 * g + 8 + r];
              hv[r] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
            }
            u32x2 pk;
            pk.x = pack_bf16x2(hv[0], hv[1]);
            pk.y = pack_bf16x2(hv[2], hv[3]);
            *reinterpret_cast<u32x2*>(orow + n) = pk;
            if (SAVE) {  // training forward: the pre-activations for the backward
              const size_t o = (size_t)p * N + n;
              u32x2 pa, pu;
              pa.x = pack_bf16x2(acc[ii][jj][4 * g], acc[ii][jj][4 * g + 1]);
              pa.y = pack_bf16x2(acc[ii][jj][4 * g + 2], acc[ii][jj][4 * g + 3]);
              pu.x = pack_bf16x2(acc[ii][jj][4 * g + 8], acc[ii][jj][4 * g + 9]);
              pu.y = pack_bf16x2(acc[ii][jj][4 * g + 10], acc[ii][jj][4 * g + 11]);
              *reinterpret_cast<u32x2*>(save_a + o) = pa;
              *reinterpret_cast<u32x2*>(save_u + o) = pu;
            }
          }
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = nb + 32 * i + 8 * g + 4 * lk;
            if (n >= N) continue;
            u32x2 pk;
            pk.x = pack_bf16x2(acc[ii][jj][4 * g], acc[ii][jj][4 * g + 1]);
            pk.y = pack_bf16x2(acc[ii][jj][4 * g + 2], acc[ii][jj][4 * g + 3]);
            *reinterpret_cast<u32x2*>(orow + n) = pk;
          }
        }
      }
    }
  };
  // (run is called straight from the switch: a lambda around it makes the
  // compiler treat the copy operands as divergent)
  switch (jn) {
    case 1: { using Q = JnSel<1, JMAX, WF>; run(typename Q::N(), typename Q::P()); } break;
    case 2: { using Q = JnSel<2, JMAX, WF>; run(typename Q::N(), typename Q::P()); } break;
    case 3: { using Q = JnSel<3, JMAX, WF>; run(typename Q::N(), typename Q::P()); } break;
    case 4: { using Q = JnSel<4, JMAX, WF>; run(typename Q::N(), typename Q::P()); } break;
    case 5: { using Q = JnSel<5, JMAX, WF>; run(typename Q::N(), typename Q::P()); } break;
    case 6: { using Q = JnSel<6, JMAX, WF>; run(typename Q::N(), typename Q::P()); } break;
    case 7: { using Q = JnSel<7, JMAX, WF>; run(typename Q::N(), typename Q::P()); } break;
    case 8: { using Q = JnSel<8, JMAX, WF>; run(typename Q::N(), typename Q::P()); } break;
    case 9: { using Q = JnSel<9, JMAX, WF>; run(typename Q::N(), typename Q::P()); } break;
    default: { using Q = JnSel<JMAX, JMAX, WF>; run(typename Q::N(), typename Q::P()); } break;
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

// Tile order: largest tiles first for layers of few experts, whose few tiles
// per block make the end of the static schedule uneven; expert order for many
// experts, where the mix of tile kinds keeps the HBM load even (measured on
// the E=8/16 and E=64/256 workloads).
constexpr int kSizedMaxExperts = 16;

template <bool GATED, int JMAX, int WF, bool GATHER, bool SAVE>
static hipError_t launch_packed_t(const moe_config& c, const void* act, const int32_t* offs,
                                  const void* wp, void* out, const int32_t* src_of,
                                  void* save_a, void* save_u, int N, int K, hipStream_t st) {
  const long rows = (long)c.T * c.k;
  const PackGeom g = pack_geom(N, K, GATED);
  // one block per CU, never more blocks than the worst-case tile count
  const long worst = (long)g.slabs * (WF == 2 ? 1 : 2) * worst_row_tiles(rows, c.E, 32 * JMAX);
  const long cap = ((long)device_cus() + 7) / 8 * 8;
  const int blocks = (int)std::min(cap, (worst + 7) / 8 * 8);
  grouped_gemm_packed_kernel<GATED, JMAX, WF, GATHER, SAVE><<<blocks, 256, 0, st>>>(
      static_cast<const uint16_t*>(act), offs, static_cast<const u32x4*>(wp),
      static_cast<uint16_t*>(out), c.E, N, K, (int)rows, g.slabs, 8,
      /*sized=*/c.E <= kSizedMaxExperts, src_of, c.k, c.T, static_cast<uint16_t*>(save_a),
      static_cast<uint16_t*>(save_u));
  return hipGetLastError();
}

// Tile shape.  Whole-slab tiles of up to 256 rows (WF = 2, JMAX = 8) unless
// they are too few to fill the chip twice over -- the down projection of a
// few experts with some hundred rows each: then half-slab tiles of up to 320
// rows (WF = 1, JMAX = 10), which double the tile count and cover an expert of
// up to 320 rows with one tile.
// N output features over a k extent of K: (f, d) for the gate / up
// projection, (d, f) for the down projection; others for the plain products
// of the backward.
template <bool GATED, bool GATHER, bool SAVE = false>
static hipError_t launch_packed(const moe_config& c, const void* act, const int32_t* offs,
                                const void* wp, void* out, const int32_t* src_of,
                                hipStream_t st, void* save_a = nullptr, void* save_u = nullptr,
                                int N = 0, int K = 0) {
  if (N == 0) {
    N = GATED ? c.f : c.d;
    K = GATED ? c.d : c.f;
  }
  const long rows = (long)c.T * c.k;
  const PackGeom g = pack_geom(N, K, GATED);
  const long typical = (long)g.slabs * std::max<long>(c.E, (rows + 255) / 256);
  if (typical < 2L * device_cus())
    return launch_packed_t<GATED, 10, 1, GATHER, SAVE>(c, act, offs, wp, out, src_of, save_a,
                                                       save_u, N, K, st);
  return launch_packed_t<GATED, 8, 2, GATHER, SAVE>(c, act, offs, wp, out, src_of, save_a, save_u,
                                                    N, K, st);
}

hipError_t launch_ffn_gate_up_packed(const moe_config& c, const void* x_perm, const int32_t* offs,
                                     const void* pgu, void* h, hipStream_t st) {
  return launch_packed<true, false>(c, x_perm, offs, pgu, h, nullptr, st);
}

hipError_t launch_ffn_gate_up_packed_gather(const moe_config& c, const void* x,
                                            const int32_t* src_of, const int32_t* offs,
                                            const void* pgu, void* h, hipStream_t st) {
  return launch_packed<true, true>(c, x, offs, pgu, h, src_of, st);
}

hipError_t launch_ffn_gate_up_packed_save(const moe_config& c, const void* act,
                                          const int32_t* src_of, const int32_t* offs,
                                          const void* pgu, void* h, void* a, void* u,
                                          hipStream_t st) {
  if (src_of) return launch_packed<true, true, true>(c, act, offs, pgu, h, src_of, st, a, u);
  return launch_packed<true, false, true>(c, act, offs, pgu, h, nullptr, st, a, u);
}

// out[rows, N] = act[rows, K] W'_e^T on a plain image of W' [E, N, K]
// (pack_geom(N, K, false)); act rows are K long.
hipError_t launch_packed_linear(const moe_config& c, const void* act, const int32_t* offs,
                                const void* wp, void* out, int N, int K, hipStream_t st) {
  return launch_packed<false, false>(c, act, offs, wp, out, nullptr, st, nullptr, nullptr, N, K);
}

hipError_t launch_pack_weights_t(const moe_config& c, const void* w_gate, const void* w_up,
                                 const void* w_down, void* packed_dh, void* packed_dx,
                                 hipStream_t st) {
  const int threads = 256, blocks = 4096;
  if (packed_dh) {
    const PackGeom g = pack_geom(c.f, c.d, false);
    const size_t total = (size_t)c.E * g.expert_elems / 8;
    pack_weights_t_kernel<<<blocks, threads, 0, st>>>(
        static_cast<const uint16_t*>(w_down), nullptr, static_cast<u32x4*>(packed_dh), c.f, c.d,
        c.d, g.slabs, g.kp, total);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (packed_dx) {
    const PackGeom g = pack_geom(c.d, 2 * c.f, false);
    const size_t total = (size_t)c.E * g.expert_elems / 8;
    pack_weights_t_kernel<<<blocks, threads, 0, st>>>(
        static_cast<const uint16_t*>(w_gate), static_cast<const uint16_t*>(w_up),
        static_cast<u32x4*>(packed_dx), c.d, c.f, 2 * c.f, g.slabs, g.kp, total);
  }
  return hipGetLastError();
}

hipError_t launch_ffn_down_packed(const moe_config& c, const void* h, const int32_t* offs,
                                  const void* pd, void* y, hipStream_t st) {
  return launch_packed<false, false>(c, h, offs, pd, y, nullptr, st);
}

}  // namespace moe
