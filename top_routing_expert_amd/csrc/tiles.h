// Device-side placement of a grouped-GEMM block on its tile.
//
// The per-expert row counts live only on the device (expert_offsets), so the
// grid is sized on the host for the worst case and every block finds its tile
// here.  Pages: [SyncTax] §2.2 (skewed expert load must not stall the rest;
// hot experts simply own more tiles) and [EP-V4] §5.2 (expert weights are
// contiguous and in expert-ID order, so neighbouring tiles share weight rows).
#pragma once

#include "common.h"

namespace moe {

// Row tiles of TM rows over every expert: sum_e ceil(c_e / TM), reduced over
// ONE whole wave (every lane gets the total).  A malformed table is clamped
// into [0, rows] so that every access stays in bounds.
template <int TM>
__device__ __forceinline__ int count_row_tiles(const int32_t* __restrict__ offs, int E, int rows,
                                               int lane) {
  int total = 0;
  for (int b0 = 0; b0 < E; b0 += 64) {
    const int e = b0 + lane;
    int nt = 0;
    if (e < E) {
      const int o0 = min(max(offs[e], 0), rows), o1 = min(max(offs[e + 1], o0), rows);
      nt = (o1 - o0 + TM - 1) / TM;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) nt += __shfl_xor(nt, o);
    total += nt;
  }
  return total;
}

// The tiles of one expert, located inside its own range: bands of up to
// `band` row tiles, inside a band by weight tile with the row tiles fastest,
// so that neighbouring tiles share the expert's weight rows (across row
// tiles) and token rows (across weight tiles).  The expert's rows are split
// evenly over its row tiles (sizes differ by at most one row): the tiles of
// one weight tile then run at the same pace side by side, and the second
// reads the weights from L2.
__device__ __forceinline__ void expert_tile(int e, int o0, int o1, int mt, int n_tiles, int band,
                                            int r, int* s_tile) {
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
  const long c = o1 - o0;
  s_tile[0] = e;
  s_tile[1] = o0 + (int)((long)m * c / mt);
  s_tile[2] = o0 + (int)((long)(m + 1) * c / mt);
  s_tile[3] = n;
}

// Finds tile L (0 <= L < row tiles * n_tiles) in the tile order, called by ONE
// whole wave.  Experts are taken in index order, or -- `sized` -- by the
// 32-row fragments of their tiles, largest first (then by index): a static
// schedule then hands out the long tiles before the short ones, so the short
// ones even out the per-block totals at the end.  (Index order mixes tiles
// that stream their own weights with tiles that share them through L2, which
// spreads the HBM load evenly over a long run of tiles.)
// Writes s_tile = {expert, first row, end row, weight tile} of the tile.
template <int TM>
__device__ __forceinline__ void locate_tile(const int32_t* __restrict__ offs, int E, int rows,
                                            int n_tiles, int band, int L, int lane, int* s_tile,
                                            bool sized = false) {
  int carry = 0;  // tiles before the current chunk of experts
  for (int cls = sized ? TM / 32 : 0; cls >= 0; --cls) {
    for (int b0 = 0; b0 < E; b0 += 64) {
      const int e = b0 + lane;
      int o0 = 0, o1 = 0;
      if (e < E) {
        o0 = min(max(offs[e], 0), rows);
        o1 = min(max(offs[e + 1], o0), rows);
      }
      const int mt = (o1 - o0 + TM - 1) / TM;
      // fragments of the expert's largest tile (0 for an empty expert)
      const int fr = mt > 0 ? ((o1 - o0 + mt - 1) / mt + 31) / 32 : 0;
      const bool in = mt > 0 && (!sized || fr == cls);
      const int cnt = in ? mt * n_tiles : 0;
      int incl = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      const int excl = carry + incl - cnt;
      if (in && L >= excl && L < excl + cnt) expert_tile(e, o0, o1, mt, n_tiles, band, L - excl, s_tile);
      carry += __shfl(incl, 63);
      if (carry > L) return;  // wave-uniform: the tile is in this chunk
    }
  }
}

// Expert-order tile table of a persistent block, built once per launch by ONE
// whole wave: for every expert its row range [o0, o1) (clamped as above) and
// the number of tiles before it (`start`, non-decreasing).  Returns the total
// tile count.  Locating a tile is then a search over LDS (locate_in_table)
// instead of a walk over the offsets in global memory.
constexpr int kTileTableMax = 1024;  // experts the table holds (every E accepted)
template <int TM>
__device__ __forceinline__ int build_tile_table(const int32_t* __restrict__ offs, int E, int rows,
                                                int n_tiles, int lane, int* t_o0, int* t_o1,
                                                int* t_start) {
  int carry = 0;
  for (int b0 = 0; b0 < E; b0 += 64) {
    const int e = b0 + lane;
    int o0 = 0, o1 = 0;
    if (e < E) {
      o0 = min(max(offs[e], 0), rows);
      o1 = min(max(offs[e + 1], o0), rows);
    }
    const int cnt = (o1 - o0 + TM - 1) / TM * n_tiles;
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (e < E) {
      t_o0[e] = o0;
      t_o1[e] = o1;
      t_start[e] = carry + incl - cnt;
    }
    carry += __shfl(incl, 63);
  }
  return carry;
}

// Tile L (0 <= L < total) of the table, expert order: its expert is the last
// one whose start is <= L (empty experts before it share its start, those
// after it start past L), found by counting with ballots.  ONE whole wave.
template <int TM>
__device__ __forceinline__ void locate_in_table(const int* t_o0, const int* t_o1,
                                                const int* t_start, int E, int n_tiles, int band,
                                                int L, int lane, int* s_tile) {
  int n = 0;
  for (int b0 = 0; b0 < E; b0 += 64) {
    const int e = b0 + lane;
    const int c = __popcll(__ballot(e < E && t_start[e] <= L));
    n += c;
    if (c < 64) break;  // wave-uniform: start is non-decreasing
  }
  const int e = max(n - 1, 0);
  if (lane == 0) {
    const int o0 = t_o0[e], o1 = t_o1[e];
    expert_tile(e, o0, o1, (o1 - o0 + TM - 1) / TM, n_tiles, band, L - t_start[e], s_tile);
  }
}

// One block per tile of a grid sized for the worst case, called by ONE whole
// wave.  The actual tile count (known only on the device) is dealt to the 8
// XCDs (the hardware hands blocks to XCDs round-robin) in equal contiguous
// ranges, so the tiles running at once on one XCD are neighbours in the tile
// order and share weight and token rows in that XCD's L2, and the surplus
// blocks of the worst-case grid never pile up on one XCD.  s_tile[0] = -1
// when the block has no tile.
template <int TM>
__device__ __forceinline__ void place_tile(const int32_t* __restrict__ offs, int E, int rows,
                                           int n_tiles, int band, int lane, int* s_tile) {
  if (lane == 0) s_tile[0] = -1;
  const int n_total = count_row_tiles<TM>(offs, E, rows, lane) * n_tiles;
  const int per_xcd = (n_total + 7) >> 3;
  const int L = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= per_xcd || L >= n_total) return;
  locate_tile<TM>(offs, E, rows, n_tiles, band, L, lane, s_tile);
}

// Upper bound of sum_e ceil(c_e / TM) over every row table with `rows` rows.
inline long worst_row_tiles(long rows, int E, int tm) {
  const long m = (rows + (long)E * (tm - 1)) / tm;
  return m < 1 ? 1 : m;
}

}  // namespace moe
