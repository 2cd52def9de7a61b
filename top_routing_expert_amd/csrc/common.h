// Shared device helpers and the internal launch interface of libmoe_mi355x.
// gfx950 (CDNA4) only: wave64, MFMA bf16 32x32x16, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Largest expert count the entry points accept (checked on the host).
constexpr int kMaxExperts = 1024;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// Raw 16-byte vector.  A native vector type (not HIP's uint4 struct) so that
// arrays of them are kept in registers by the compiler.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 helpers
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ------------------------------------------------------------ ordering keys
// Maps a float to a uint32 whose unsigned order is the float order (finite
// values; -0 must have been canonicalised to +0 before).
__device__ __forceinline__ uint32_t ord_key(float s) {
  uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------ launch helpers
inline int div_up(long a, long b) { return (int)((a + b - 1) / b); }

// ------------------------------------------------------------ internal launches
// Every launcher returns hipSuccess or the launch error; shapes are validated
// by the C-ABI layer before these are called.
hipError_t launch_router_gemm_bf16(const uint16_t* x, const uint16_t* wr, float* dst, int T, int d,
                                   int E, int splits, hipStream_t st);
hipError_t launch_router_gemm_f32(const float* x, const float* wr, float* dst, int T, int d, int E,
                                  hipStream_t st);
hipError_t launch_topk(const moe_config& c, const float* partial, int splits, const float* bias,
                       float* logits_out, int32_t* topk_idx, float* topk_w, hipStream_t st);
int router_splits(const moe_config& c);

hipError_t launch_permute(const moe_config& c, const void* x, const int32_t* topk_idx,
                          int32_t* expert_offsets, int32_t* rank_offsets, int32_t* slot_of,
                          int32_t* src_of, void* x_perm, void* ws, hipStream_t st);
size_t permute_ws_bytes(const moe_config& c);
// The allocation-free permute's static scratch: its size, and the current
// device's address of it (looked up once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
hipError_t noalloc_scratch(void** ptr);

hipError_t launch_ffn_gate_up(const moe_config& c, const void* x_perm, const int32_t* offs,
                              const void* wg, const void* wu, void* h, hipStream_t st);
hipError_t launch_ffn_down(const moe_config& c, const void* h, const int32_t* offs, const void* wd,
                           void* y, hipStream_t st);

// Packed expert weights (MFMA fragment order, zero padded; see ffn_packed.hip).
struct PackGeom {
  int slab_features;    // output features per slab (128 gated, 256 plain)
  int slabs;            // slabs per expert
  int kp;               // K rounded up to the 128-wide k iteration
  size_t expert_elems;  // bf16 elements per expert
};
PackGeom pack_geom(int features, int K, bool gated);
hipError_t launch_pack_weights(const moe_config& c, const void* wg, const void* wu, const void* wd,
                               void* packed_gate_up, void* packed_down, hipStream_t st);
hipError_t launch_ffn_gate_up_packed(const moe_config& c, const void* x_perm, const int32_t* offs,
                                     const void* packed_gate_up, void* h, hipStream_t st);
hipError_t launch_ffn_gate_up_packed_gather(const moe_config& c, const void* x,
                                            const int32_t* src_of, const int32_t* offs,
                                            const void* pgu, void* h, hipStream_t st);
// gate/up with the pre-activations a = x Wg^T and u = x Wu^T also written
// (bf16, [rows, f]); src_of != NULL gathers the rows from token order.
hipError_t launch_ffn_gate_up_packed_save(const moe_config& c, const void* act,
                                          const int32_t* src_of, const int32_t* offs,
                                          const void* pgu, void* h, void* a, void* u,
                                          hipStream_t st);
// out[rows, N] = act[rows, K] W'_e^T on a plain packed image of W' [E, N, K].
hipError_t launch_packed_linear(const moe_config& c, const void* act, const int32_t* offs,
                                const void* wp, void* out, int N, int K, hipStream_t st);
// Plain packed images of W_d^T (N = f, K = d) and [W_g; W_u]^T (N = d, K = 2 f).
hipError_t launch_pack_weights_t(const moe_config& c, const void* w_gate, const void* w_up,
                                 const void* w_down, void* packed_dh, void* packed_dx,
                                 hipStream_t st);
hipError_t launch_ffn_down_packed(const moe_config& c, const void* h, const int32_t* offs,
                                  const void* packed_down, void* y, hipStream_t st);

size_t route_stats_ws_bytes(const moe_config& c);
hipError_t launch_route_stats(const moe_config& c, const float* logits, const float* bias,
                              const int32_t* offs, const int32_t* roffs, int32_t* hist,
                              int32_t* rank_load, float* stats, void* ws, hipStream_t st);
bool fp8_row_supported(const moe_config& c);
hipError_t launch_fp8_quantize(const moe_config& c, const void* x, void* codes, float* scale_zero,
                               hipStream_t st);
hipError_t launch_fp8_dequantize(const moe_config& c, const void* codes, const int32_t* src_of,
                                 const float* scale_zero, void* x_perm, hipStream_t st);
// FP8 first GEMM (ffn_fp8.hip): the weight image's geometry, its packing
// and the gather GEMM on per-token FP8 codes.
struct Fp8Geom {
  long rows;           // packed rows per expert (2 f: gate and up)
  size_t codes_bytes;  // E * rows * d
  size_t scale_off;    // byte offset of the per-row scales
  size_t csum_off;     // byte offset of the per-row code sums
  size_t total;        // image bytes
};
Fp8Geom fp8_geom(const moe_config& c);
hipError_t launch_pack_weights_fp8(const moe_config& c, const void* wg, const void* wu,
                                   void* image, hipStream_t st);
hipError_t launch_ffn_gate_up_fp8_gather(const moe_config& c, const void* x_codes,
                                         const float* scale_zero, const int32_t* src_of,
                                         const int32_t* offs, const void* image, void* h,
                                         hipStream_t st);
// topk_idx != NULL and wave >= 0 (bf16 only): combine only the tokens whose
// highest-numbered chosen expert is in experts [wave * per, (wave + 1) * per).
hipError_t launch_combine(const moe_config& c, const void* y_perm, const int32_t* slot_of,
                          const float* topk_w, void* out, hipStream_t st,
                          const int32_t* topk_idx = nullptr, int wave = -1, int per = 1);

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t st);

// Layer backward (backward.hip); bf16 only.
hipError_t launch_grouped_linear(const moe_config& c, const uint16_t* act, const int32_t* offs,
                                 const uint16_t* w, uint16_t* out, int N, int K, hipStream_t st);
hipError_t launch_combine_backward(const moe_config& c, const void* d_out, const void* y_perm,
                                   const int32_t* slot_of, const float* topk_w, void* d_y_perm,
                                   float* d_topk_w, hipStream_t st);
size_t ffn_backward_ws_bytes(const moe_config& c);
hipError_t launch_ffn_backward(const moe_config& c, const void* x_perm, const int32_t* offs,
                               const void* wg, const void* wu, const void* wd, const void* a_in,
                               const void* u_in, const void* packed_dh, const void* packed_dx,
                               const void* d_y_perm, void* d_x_perm, void* d_wg, void* d_wu,
                               void* d_wd, void* ws, hipStream_t st);
size_t route_backward_ws_bytes(const moe_config& c);
hipError_t launch_route_backward(const moe_config& c, const void* x, const void* w_router,
                                 const float* logits, const float* bias, const int32_t* topk_idx,
                                 const float* d_topk_w, float* d_logits, void* d_x_router,
                                 void* d_w_router, float* d_bias, void* ws, hipStream_t st);
hipError_t launch_unpermute_backward(const moe_config& c, const void* d_x_perm,
                                     const int32_t* slot_of, const void* d_x_router, void* d_x,
                                     hipStream_t st);

}  // namespace moe
