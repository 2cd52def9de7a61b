// Dispatch layout: per-expert histogram, exclusive scan, stable permutation
// and the row copy x -> x_perm.
//
// Pages: [ThunderEP] §2 (T*k expert calls per batch); [EP-V4] §3.3 (rows
// packed per destination, one chunk per expert in expert-ID order, so a
// receiver indexes them directly), §3.1 (contiguous expert blocks per
// machine), §5.5 (256-byte aligned packed buffers: every row here is d
// elements, d a multiple of 64, i.e. >= 128 bytes and 16-byte aligned).
//
// gfx950 design (deterministic, no atomics on global memory):
//  1. count : one block per chunk of 256 tokens (one thread per token).  Each
//     wave ORs its lane bit into a per-wave LDS bitmask per expert; a pair's
//     rank inside the chunk is the popcount of the earlier waves' masks plus
//     the popcount of its own wave's mask below its lane.  Since a token picks
//     an expert at most once, this is exactly "earlier tokens of the chunk
//     routed to e".  Writes the per-chunk counts and each pair's chunk rank.
//  2. scan  : one block turns the per-chunk counts into per-chunk bases
//     (exclusive over chunks) and the totals into expert_offsets and
//     rank_offsets.  Batches of at most four chunks (E <= 256) run 1 and 2
//     as one block (one launch fewer; for more chunks the parallel count
//     blocks win).
//  3. scatter: one wave per token computes its k slots, writes slot_of /
//     src_of, reads the token row once and stores it to its k slots with
//     16-byte vector accesses (x is read once; x_perm written once).  With no
//     x_perm it writes the indices only.
#include <mutex>

#include "common.h"

namespace moe {

constexpr int kChunk = 256;
constexpr int kMaxK = 16;

__global__ __launch_bounds__(256) void perm_count_kernel(const int32_t* __restrict__ topk_idx, int T,
                                                         int k, int E, int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ rank) {
  extern __shared__ unsigned long long masks[];  // [4][E]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < 4 * E; i += 256) masks[i] = 0ull;
  __syncthreads();
  const int t = blockIdx.x * kChunk + tid;
  int ev[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    ev[j] = 0;
    if (j < k && t < T) {
      int e = topk_idx[(size_t)t * k + j];
      e = e < 0 ? 0 : (e >= E ? E - 1 : e);  // keep every access in bounds
      ev[j] = e;
      atomicOr(&masks[w * E + e], 1ull << lane);
    }
  }
  __syncthreads();
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k && t < T) {
      const int e = ev[j];
      int r = __popcll(masks[w * E + e] & below);
      for (int v = 0; v < w; ++v) r += __popcll(masks[v * E + e]);
      rank[(size_t)t * k + j] = r;
    }
  }
  for (int e = tid; e < E; e += 256) {
    int c = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) c += __popcll(masks[v * E + e]);
    counts[(size_t)blockIdx.x * E + e] = c;
  }
}

// Exclusive scan of the per-expert totals over the experts (one block of 1024
// threads; thread e < E holds expert e's total) -> expert_offsets [E + 1] and
// rank_offsets [R + 1].
__device__ __forceinline__ void scan_expert_totals(int total, int E, int R,
                                                   int32_t* __restrict__ expert_offsets,
                                                   int32_t* __restrict__ rank_offsets,
                                                   int32_t* s_excl, int32_t* s_wave) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int incl = total;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) s_wave[w] = incl;
  __syncthreads();
  if (w == 0) {
    int wv = lane < 16 ? s_wave[lane] : 0;
    int wi = wv;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int y = __shfl_up(wi, o);
      if (lane >= o) wi += y;
    }
    if (lane < 16) s_wave[lane] = wi - wv;  // exclusive wave bases
  }
  __syncthreads();
  const int excl = s_wave[w] + incl - total;
  if (tid < E) s_excl[tid] = excl;
  if (tid == E - 1) s_excl[E] = excl + total;
  __syncthreads();
  if (tid < E) expert_offsets[tid] = s_excl[tid];
  if (tid < R) rank_offsets[tid] = s_excl[tid * (E / R)];
  if (tid == 0) {
    expert_offsets[E] = s_excl[E];
    rank_offsets[R] = s_excl[E];
  }
}

// counts[c][e] -> exclusive base over chunks (in place); totals -> offsets.
__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t* __restrict__ counts, int nchunk,
                                                         int E, int R,
                                                         int32_t* __restrict__ expert_offsets,
                                                         int32_t* __restrict__ rank_offsets) {
  __shared__ int32_t s_excl[1025];
  __shared__ int32_t s_wave[16];
  const int tid = threadIdx.x;
  int total = 0;
  if (tid < E) {
    constexpr int B = 16;
    for (int c0 = 0; c0 < nchunk; c0 += B) {
      int v[B];
#pragma unroll
      for (int u = 0; u < B; ++u) v[u] = (c0 + u < nchunk) ? counts[(size_t)(c0 + u) * E + tid] : 0;
#pragma unroll
      for (int u = 0; u < B; ++u) {
        if (c0 + u < nchunk) counts[(size_t)(c0 + u) * E + tid] = total;
        total += v[u];
      }
    }
  }
  scan_expert_totals(total, E, R, expert_offsets, rank_offsets, s_excl, s_wave);
}

// Small batches (at most kFusedChunks chunks, E <= kFusedMaxE): count and scan
// in one block of 1024 threads, four chunks per pass (four waves per chunk,
// exactly as perm_count_kernel), the per-chunk counts kept in LDS.  Writes the
// same outputs as perm_count_kernel followed by perm_scan_kernel.  The kernel
// handles any number of passes; it is launched for one.
constexpr int kFusedChunks = 4;
constexpr int kFusedMaxE = 256;

__global__ __launch_bounds__(1024) void perm_count_scan_kernel(
    const int32_t* __restrict__ topk_idx, int T, int k, int E, int R, int nchunk,
    int32_t* __restrict__ base, int32_t* __restrict__ rank, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ rank_offsets) {
  extern __shared__ unsigned long long masks[];  // [16 waves][E], then int32 cnt[nchunk][E]
  int32_t* cnt = reinterpret_cast<int32_t*>(masks + 16 * E);
  __shared__ int32_t s_excl[kFusedMaxE + 1];
  __shared__ int32_t s_wave[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int cw = w & 3, cs = w >> 2;  // wave inside its chunk, chunk inside the pass
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int c0 = 0; c0 < nchunk; c0 += 4) {
    for (int i = tid; i < 16 * E; i += 1024) masks[i] = 0ull;
    __syncthreads();
    const int c = c0 + cs;
    const int t = c * kChunk + (tid & (kChunk - 1));
    const bool live = c < nchunk && t < T;
    int ev[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      ev[j] = 0;
      if (j < k && live) {
        int e = topk_idx[(size_t)t * k + j];
        e = e < 0 ? 0 : (e >= E ? E - 1 : e);  // keep every access in bounds
        ev[j] = e;
        atomicOr(&masks[w * E + e], 1ull << lane);
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k && live) {
        const int e = ev[j];
        int r = __popcll(masks[w * E + e] & below);
        for (int v = 0; v < cw; ++v) r += __popcll(masks[(cs * 4 + v) * E + e]);
        rank[(size_t)t * k + j] = r;
      }
    }
    for (int i = tid; i < 4 * E; i += 1024) {
      const int sl = i / E, e = i - sl * E;
      if (c0 + sl < nchunk) {
        int n = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) n += __popcll(masks[(sl * 4 + v) * E + e]);
        cnt[(c0 + sl) * E + e] = n;
      }
    }
    __syncthreads();  // masks are cleared by the next pass
  }
  int total = 0;
  if (tid < E) {
    for (int c = 0; c < nchunk; ++c) {
      base[(size_t)c * E + tid] = total;
      total += cnt[c * E + tid];
    }
  }
  scan_expert_totals(total, E, R, expert_offsets, rank_offsets, s_excl, s_wave);
}

__global__ __launch_bounds__(256) void perm_scatter_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ rank, const int32_t* __restrict__ base,
    const int32_t* __restrict__ expert_offsets, int T, int k, int E, int row_vecs,
    int32_t* __restrict__ slot_of, int32_t* __restrict__ src_of, u32x4* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave
  int p = 0;
  if (lane < k) {
    int e = topk_idx[(size_t)t * k + lane];
    e = e < 0 ? 0 : (e >= E ? E - 1 : e);
    p = expert_offsets[e] + base[(size_t)(t / kChunk) * E + e] + rank[(size_t)t * k + lane];
    slot_of[(size_t)t * k + lane] = p;
    src_of[p] = t * k + lane;
  }
  if (!x_perm) return;  // index outputs only (the first GEMM gathers the rows)
  int pj[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) pj[j] = __shfl(p, j);
  const u32x4* src = x + (size_t)t * row_vecs;
  for (int v = lane; v < row_vecs; v += 4 * 64) {
    u32x4 val[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (v + u * 64 < row_vecs) val[u] = src[v + u * 64];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        u32x4* dst = x_perm + (size_t)pj[j] * row_vecs;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (v + u * 64 < row_vecs) dst[v + u * 64] = val[u];
      }
    }
  }
}

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t permute_ws_bytes(const moe_config& c) {
  const size_t nchunk = (size_t)div_up(c.T, kChunk);
  return align256(nchunk * c.E * sizeof(int32_t)) + align256((size_t)c.T * c.k * sizeof(int32_t));
}

hipError_t launch_permute(const moe_config& c, const void* x, const int32_t* topk_idx,
                          int32_t* expert_offsets, int32_t* rank_offsets, int32_t* slot_of,
                          int32_t* src_of, void* x_perm, void* ws, hipStream_t st) {
  const int nchunk = div_up(c.T, kChunk);
  int32_t* counts = static_cast<int32_t*>(ws);
  int32_t* rank = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                             align256((size_t)nchunk * c.E * sizeof(int32_t)));
  hipError_t err;
  if (nchunk <= kFusedChunks && c.E <= kFusedMaxE) {
    const size_t lds = 16 * (size_t)c.E * sizeof(unsigned long long) +
                       (size_t)nchunk * c.E * sizeof(int32_t);
    perm_count_scan_kernel<<<1, 1024, lds, st>>>(topk_idx, c.T, c.k, c.E, c.ep_ranks, nchunk,
                                                 counts, rank, expert_offsets, rank_offsets);
    err = hipGetLastError();
  } else {
    perm_count_kernel<<<nchunk, 256, 4 * c.E * sizeof(unsigned long long), st>>>(
        topk_idx, c.T, c.k, c.E, counts, rank);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    perm_scan_kernel<<<1, 1024, 0, st>>>(counts, nchunk, c.E, c.ep_ranks, expert_offsets,
                                         rank_offsets);
    err = hipGetLastError();
  }
  if (err != hipSuccess) return err;
  const int elem = c.dtype == MOE_BF16 ? 2 : 4;
  const int row_vecs = (int)((size_t)c.d * elem / 16);
  perm_scatter_kernel<<<div_up(c.T, 4), 256, 0, st>>>(
      static_cast<const u32x4*>(x), topk_idx, rank, counts, expert_offsets, c.T, c.k, c.E, row_vecs,
      slot_of, src_of, static_cast<u32x4*>(x_perm));
  return hipGetLastError();
}

// ------------------------------------------------- allocation-free scratch
// moe_permute_noalloc's scratch (the per-chunk counts and pair ranks that
// moe_permute keeps in its caller's workspace): a static device array of
// kNoAllocScratchBytes.  Every GPU the library runs on holds its own copy
// from module load until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: the device address is looked
// up once per device with hipGetSymbolAddress and only that address is used.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // the current device's copy
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace moe
