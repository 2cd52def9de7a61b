/*
 * moe.h -- C ABI of libmoe_mi355x.so: the forward token path of one
 * Mixture-of-Experts layer on one MI355X (gfx950) GPU.
 *
 *   router (gate GEMM, scores, top-k, gates)  -> moe_route
 *   histogram + stable permute (dispatch)     -> moe_permute
 *   expert SwiGLU FFN, grouped over experts   -> moe_ffn_gate_up, moe_ffn_down
 *                                                (both: moe_grouped_ffn)
 *   weighted combine back to token order      -> moe_combine
 *   all of the above in one call              -> moe_layer_fwd
 *
 * Pages cited by title and section:
 *   [EP-V4]      "DeepSeek-V4的Expert Parallelism与计算通信遮掩实战解析" (tqpw.cn)
 *   [ThunderEP]  ThunderEP article on MoE expert parallelism over PCIe
 *                (discosf.com), section 2 "MoE专家并行的通信本质"
 *   [V4-overlap] "DeepSeek-v4 Parallel comp-comm overlap" (recsys-frontier
 *                blog), sections "先让 EP 在 IB 网络上跑起来" and
 *                "V4 的 Waved-EP 通信计算遮掩"
 *   [SyncTax]    "Deepseek-MoE同步税本质与四层实战优化指南" (qwbw.cn)
 *
 * The problem is stated as in the pages: T tokens of hidden size d, E experts,
 * top-k experts per token, expert intermediate size f ([SyncTax] §2.1;
 * [ThunderEP] §2; [EP-V4] §4.2 config fields num_experts / top_k /
 * expert_parallel_size).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  Every tensor pointer is a DEVICE pointer to a dense row-major array
 *   owned by the caller; the library allocates nothing, frees nothing and
 *   keeps no pointer after a call returns.  `ws` is caller-provided device
 *   scratch of at least the size moe_workspace_bytes() reports for that entry
 *   point (it may be NULL when that size is 0).  Calls that share a `ws`
 *   buffer must not overlap in time.
 * Element types.  cfg->dtype == MOE_BF16: x, w_*, x_perm, h, y_perm and out are
 *   bfloat16 (raw 16-bit patterns); MOE_F32: all of them are float32.  Router
 *   logits, bias and gate weights are always float32; indices and offsets are
 *   int32.  Accumulation is always float32.
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 *   stream).  Every call only enqueues work and returns: no host
 *   synchronisation and no device-to-host copy.  Per-expert counts stay on the
 *   device; the grouped FFN reads expert_offsets on the device.
 * Errors.  All arguments are checked on the host before anything is launched;
 *   a failed check returns a negative status and leaves every output
 *   untouched.  A failed launch returns MOE_EHIP.  Errors raised inside a
 *   kernel surface at the caller's next synchronisation.
 * Values.  Non-finite inputs are unsupported (indices still stay in range).
 *   topk_idx handed to moe_permute must hold distinct in-range experts per
 *   token; otherwise the outputs are unspecified, but every access stays
 *   inside the buffers described here.
 * Determinism.  Every output is bitwise reproducible run to run (no
 *   floating-point atomics; fixed reduction orders).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = -1,       /* bad shape, flag, pointer or workspace size         */
  MOE_EUNSUPPORTED = -2, /* valid problem outside what the kernels implement   */
  MOE_EHIP = -3,         /* a HIP launch failed                                */
  MOE_ESCRATCH = -4      /* more scratch than the static array of the
                            allocation-free entry point holds                  */
};

enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 };

/* Which entry point a workspace size is asked for. */
enum moe_entry {
  MOE_ENTRY_ROUTE = 1,
  MOE_ENTRY_PERMUTE = 2,
  MOE_ENTRY_FFN = 3,
  MOE_ENTRY_COMBINE = 4,
  MOE_ENTRY_LAYER = 5,
  MOE_ENTRY_ROUTE_STATS = 6,
  MOE_ENTRY_FFN_BACKWARD = 7,
  MOE_ENTRY_ROUTE_BACKWARD = 8
};

/*
 * Problem description.
 *   T, d, E, k, f  tokens, hidden size, experts, experts per token, expert
 *                  intermediate size.  T may be 0 (an empty batch).
 *   n_group, topk_group
 *                  group-limited routing: experts form n_group contiguous
 *                  groups of E/n_group; a group's score is the max of its
 *                  experts' scores; only the topk_group best groups are
 *                  eligible ([V4-overlap], EP-on-IB section: 8 experts chosen
 *                  within the best 4 nodes).  n_group = topk_group = 1: off.
 *   presel         0: off.  P > 0: the softmax is taken over the P best
 *                  scores only, then the top-k of those are kept ([EP-V4]
 *                  §3.2: partial sort to the top-8, exact softmax over those).
 *   renorm         1: the k gates are renormalised to sum to 1 (softmax over
 *                  the chosen set).  0: raw softmax probabilities over the
 *                  pre-selected set (presel > 0) or over all E (presel = 0).
 *   ep_ranks       R >= 1 expert-parallel ranks of the emitted send layout;
 *                  rank r owns experts [r*E/R, (r+1)*E/R) ([EP-V4] §3.1:
 *                  experts 0-7 on machine 0, 8-15 on machine 1, ...).
 *   dtype          MOE_F32 or MOE_BF16.
 * Limits: 1 <= k <= 16, k <= E <= 1024, presel = 0 or k <= presel <= min(E, 32),
 *   n_group <= 64 divides E, topk_group*(E/n_group) >= max(k, presel),
 *   R divides E.  MOE_BF16 needs d and f multiples of 64; MOE_F32 needs d
 *   and f multiples of 4.  (T*k)*max(d, f) < 2^31.
 */
typedef struct moe_config {
  int32_t T, d, E, k, f;
  int32_t n_group, topk_group;
  int32_t presel;
  int32_t renorm;
  int32_t ep_ranks;
  int32_t dtype;
} moe_config;

/*
 * Optional caller buffers for moe_layer_fwd's intermediates (device
 * pointers).  A NULL field is carved from `ws` instead; a non-NULL field
 * receives that intermediate exactly as the corresponding stage entry point
 * would write it (routing indices kept for reuse: [SyncTax] §2.4).
 */
typedef struct moe_layer_bufs {
  float* logits;           /* [T, E]            */
  int32_t* topk_idx;       /* [T, k]            */
  float* topk_w;           /* [T, k]            */
  int32_t* expert_offsets; /* [E + 1]           */
  int32_t* rank_offsets;   /* [ep_ranks + 1]    */
  int32_t* slot_of;        /* [T * k]           */
  int32_t* src_of;         /* [T * k]           */
  void* x_perm;            /* [T * k, d]        */
  void* h;                 /* [T * k, f]        */
  void* y_perm;            /* [T * k, d]        */
} moe_layer_bufs;

/* Human-readable text of a moe_status value (static storage). */
const char* moe_strerror(int status);

/* Checks a configuration as moe_layer_fwd would; returns a moe_status. */
int moe_validate(const moe_config* cfg);

/*
 * Bytes of `ws` that entry point `entry` (enum moe_entry) needs for `cfg`,
 * written to *bytes.  For MOE_ENTRY_LAYER it assumes every moe_layer_bufs
 * field is NULL (the worst case).  Returns a moe_status.
 */
int moe_workspace_bytes(const moe_config* cfg, int entry, size_t* bytes);

/*
 * Router: gate GEMM, scores, expert selection and gate weights.
 *   z[t,e] = sum_i x[t,i] * w_router[e,i] in float32 ([EP-V4] §2.1: every
 *   token's logits over all experts, then top-k and softmax gates locally);
 *   s = z + bias[e] as one float32 add (-0 counts as +0); experts are ordered
 *   by (s descending, index ascending) within the eligible groups; the first
 *   k are written best first.  Gates: m = best score, e_j = exp(s_j - m)
 *   ([EP-V4] §3.2 max subtraction), divided by the sum over the k chosen
 *   (renorm = 1), the presel best (presel > 0) or all E experts.
 *   x         [T, d] (dtype), or NULL: then `logits` is an INPUT [T, E] float32
 *             and only selection and gates run.
 *   w_router  [E, d] (dtype); ignored when x is NULL.
 *   bias      [E] float32 or NULL (no bias).
 *   logits    [T, E] float32: output when x != NULL, input otherwise.
 *   topk_idx  [T, k] int32 out;  topk_w [T, k] float32 out.
 */
int moe_route(const moe_config* cfg, const void* x, const void* w_router, const float* bias,
              float* logits, int32_t* topk_idx, float* topk_w,
              void* ws, size_t ws_bytes, void* stream);

/*
 * Dispatch layout: per-expert histogram, exclusive scan and a stable
 * permutation of the T*k (token, choice) pairs into expert-contiguous rows.
 *   c_e = #pairs routed to e (sum = T*k: [ThunderEP] §2, 1024 tokens x top-2
 *   are 2048 expert calls); expert_offsets = exclusive prefix sum of c (E+1
 *   entries, last = T*k); the rows of expert e hold its tokens in ascending
 *   token order: p(t,j) = expert_offsets[e] + #{t' < t routed to e}.
 *   Rows are packed per destination, one chunk per expert in expert-ID order
 *   ([EP-V4] §3.3), so the buffer is also the rank-major send layout:
 *   rank r's chunk is rows [rank_offsets[r], rank_offsets[r+1]) with
 *   rank_offsets[r] = expert_offsets[r*E/R].
 *   x              [T, d] (dtype) in.   topk_idx [T, k] int32 in.
 *   expert_offsets [E+1] int32 out.     rank_offsets [R+1] int32 out.
 *   slot_of        [T*k] int32 out: slot_of[t*k+j] = p(t,j).
 *   src_of         [T*k] int32 out: src_of[p] = t*k+j (inverse of slot_of).
 *   x_perm         [T*k, d] (dtype) out: x_perm[p] = x[t], bit-exact copies.
 *   x and x_perm may both be NULL: then only the index outputs are written
 *   (for moe_ffn_gate_up_packed_gather, which reads the rows itself).
 */
int moe_permute(const moe_config* cfg, const void* x, const int32_t* topk_idx,
                int32_t* expert_offsets, int32_t* rank_offsets, int32_t* slot_of,
                int32_t* src_of, void* x_perm, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_permute_noalloc: moe_permute for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments and outputs as moe_permute, bit for bit,
 * without `ws`: the per-chunk counts and pair ranks go to a static device
 * array of moe_noalloc_scratch_bytes() bytes (16 MiB) that the library holds
 * on every GPU it runs on until the process ends.  The call allocates and
 * frees nothing; its first call on a device looks up that device's copy of
 * the array (hipGetSymbolAddress).  A problem whose scratch (about
 * 4 (ceil(T / 256) E + T k) bytes) exceeds the array returns MOE_ESCRATCH
 * before anything is launched.  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be serialised by the caller.  Nothing in the array
 * needs to start at zero: every value a call reads it has written first.
 */
int moe_permute_noalloc(const moe_config* cfg, const void* x, const int32_t* topk_idx,
                        int32_t* expert_offsets, int32_t* rank_offsets, int32_t* slot_of,
                        int32_t* src_of, void* x_perm, void* stream);

/* Bytes of the static scratch array behind moe_permute_noalloc. */
size_t moe_noalloc_scratch_bytes(void);

/*
 * Expert FFN, first half, grouped over experts: for every expert e and every
 * row p in [expert_offsets[e], expert_offsets[e+1]):
 *   h[p] = SiLU(x_perm[p] . w_gate[e]^T) * (x_perm[p] . w_up[e]^T),
 *   SiLU(a) = a / (1 + exp(-a)); float32 accumulation, h stored in dtype
 *   (bf16 rounds to nearest even).  The expert FFN is "L1 + Act + L2"
 *   ([V4-overlap], Waved-EP section); expert weights are contiguous and in
 *   expert-ID order ([EP-V4] §5.2).
 *   x_perm         [rows, d] (dtype).
 *   expert_offsets [E+1] int32 ABSOLUTE row offsets, non-decreasing, last
 *                  <= T*k.  A sub-table (expert_offsets + e0 with cfg->E set
 *                  to the number of experts of one rank and the weight
 *                  pointers advanced by e0 experts) runs exactly one rank's
 *                  share; rows outside the table are not touched.
 *   w_gate, w_up   [E, f, d] (dtype).   h [T*k, f] (dtype) out.
 * Only T, d, E, k, f and dtype of cfg are used.
 */
int moe_ffn_gate_up(const moe_config* cfg, const void* x_perm, const int32_t* expert_offsets,
                    const void* w_gate, const void* w_up, void* h, void* stream);

/*
 * Expert FFN, second half: y_perm[p] = h[p] . w_down[e]^T for the rows of
 * every expert e (same row-table rules as moe_ffn_gate_up).
 *   h [T*k, f] (dtype).  w_down [E, d, f] (dtype).  y_perm [T*k, d] (dtype) out.
 */
int moe_ffn_down(const moe_config* cfg, const void* h, const int32_t* expert_offsets,
                 const void* w_down, void* y_perm, void* stream);

/* moe_ffn_gate_up followed by moe_ffn_down on the same stream. */
int moe_grouped_ffn(const moe_config* cfg, const void* x_perm, const int32_t* expert_offsets,
                    const void* w_gate, const void* w_up, const void* w_down,
                    void* h, void* y_perm, void* stream);

/*
 * Weighted combine back to token order ([SyncTax] §2.3: each token's k expert
 * outputs summed with their gate weights on the token's home device):
 *   out[t] = sum over j = 0..k-1, in that order, of topk_w[t,j] * y_perm[slot_of[t*k+j]],
 *   float32 accumulation, stored in dtype.
 *   y_perm [T*k, d] (dtype).  slot_of [T*k] int32, each in [0, T*k).
 *   topk_w [T, k] float32.    out [T, d] (dtype) out.
 */
int moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* slot_of,
                const float* topk_w, void* out, void* stream);

/*
 * The whole layer: moe_route -> moe_permute -> moe_ffn_gate_up ->
 * moe_ffn_down -> moe_combine on one stream; dispatch, expert compute and
 * combine run serially as the method states ([V4-overlap], EP-on-IB
 * section).  `bufs` may be NULL (every intermediate lives in ws).
 *   x [T, d], w_router [E, d], bias [E] float32 or NULL,
 *   w_gate / w_up [E, f, d], w_down [E, d, f], out [T, d].
 */
int moe_layer_fwd(const moe_config* cfg, const void* x, const void* w_router, const float* bias,
                  const void* w_gate, const void* w_up, const void* w_down, void* out,
                  const moe_layer_bufs* bufs, void* ws, size_t ws_bytes, void* stream);

/*
 * Packed expert weights (MOE_BF16 only).
 *
 * The expert weights are static across forward passes, so they can be laid
 * out once, at load time, in the order the grouped-GEMM kernels consume them:
 * each expert's image is a sequence of 1 KB blocks, one per wave load, in the
 * matrix cores' operand order, zero padded to whole tiles.  The packed FFN
 * computes exactly what moe_ffn_gate_up / moe_ffn_down compute ([V4-overlap]
 * Waved-EP section, expert compute = L1 + Act + L2), with the weights read
 * straight from HBM into registers instead of through LDS.  Each expert's
 * image is contiguous and in expert-ID order ([EP-V4] §5.2), so one rank's
 * share is still a plain offset: expert e0's image starts at byte
 * e0 * (gate_up_bytes / E) (resp. down_bytes / E).
 *
 * moe_packed_weight_bytes: bytes of the two packed images for cfg (T, k and
 *   the routing fields are ignored).  Fails with MOE_EUNSUPPORTED unless
 *   dtype is MOE_BF16.
 * moe_pack_weights: writes packed_gate_up from w_gate and w_up ([E, f, d]),
 *   and/or packed_down from w_down ([E, d, f]); either output may be NULL (its
 *   inputs are then ignored).  All pointers 16-byte aligned.  Enqueue-only,
 *   like every other call.
 */
int moe_packed_weight_bytes(const moe_config* cfg, size_t* gate_up_bytes, size_t* down_bytes);
int moe_pack_weights(const moe_config* cfg, const void* w_gate, const void* w_up,
                     const void* w_down, void* packed_gate_up, void* packed_down, void* stream);

/*
 * moe_ffn_gate_up / moe_ffn_down / moe_layer_fwd on packed weights: same
 * arguments, same outputs (h, y_perm, out within the same float32
 * accumulation; the sums run over k in the same order), same row-table and
 * sub-table rules.  x_perm, h and y_perm must be 16-byte aligned.
 */
int moe_ffn_gate_up_packed(const moe_config* cfg, const void* x_perm,
                           const int32_t* expert_offsets, const void* packed_gate_up, void* h,
                           void* stream);
int moe_ffn_down_packed(const moe_config* cfg, const void* h, const int32_t* expert_offsets,
                        const void* packed_down, void* y_perm, void* stream);

/*
 * Routing diagnostics of one batch: the load-balance report of [SyncTax] §5.1
 * (per-expert activation frequency; the entropy of the routing, ideal log2 E
 * bits) and [EP-V4] §6.2 (per-expert activation shares, ideal 1/E).
 *   logits         [T, E] fp32 in: z as moe_route wrote it (before the bias).
 *   bias           [E] fp32 in or NULL (the same as for moe_route).
 *   expert_offsets [E+1], rank_offsets [R+1] int32 in: from moe_permute.
 *   hist           [E] int32 out: (token, choice) pairs per expert.
 *   rank_load      [R] int32 out: pairs per rank (contiguous blocks of E/R).
 *   stats          [4] fp32 out:
 *     [0] mean over tokens of -sum_e p_e log2 p_e, p = softmax over all E
 *         experts of the fp32 scores s = z + b;
 *     [1] mean over tokens of the softmax mass outside the presel experts
 *         ranked first by (s desc, e asc) -- what the partial softmax over
 *         the pre-selection leaves out; 0 when presel = 0;
 *     [2] -sum_e q_e log2 q_e, q = hist / (T k), zero shares dropped;
 *     [3] E * max_e hist[e] / (T k) (1 = perfectly even).
 *   ws: moe_workspace_bytes(MOE_ENTRY_ROUTE_STATS).  T = 0 writes zeros.
 *   The sums run in a fixed order: the report is bitwise reproducible.
 */
int moe_route_stats(const moe_config* cfg, const float* logits, const float* bias,
                    const int32_t* expert_offsets, const int32_t* rank_offsets, int32_t* hist,
                    int32_t* rank_load, float* stats, void* ws, size_t ws_bytes, void* stream);

/*
 * Per-token FP8 compression of the dispatch payload ([SyncTax] §3.1: the
 * token vectors that cross the all-to-all are quantised to FP8 with their own
 * min / max and an affine map, one byte per element).  bf16, d <= 8192.
 * moe_quantize_fp8 (sender): for every token t,
 *   z = (max_i x[t,i] + min_i x[t,i]) / 2, s = ((max - min) / 2) / 448 (float32),
 *   codes[t,i] = E4M3((x[t,i] - z) / s), clamped to +-448, rounded to nearest
 *   (ties to the even code); a constant row gets s = 0 and codes 0.
 *   x [T, d] bf16 in; codes [T, d] uint8 out; scale_zero [T, 2] fp32 out (s, z).
 *   E4M3: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, largest 448.
 * moe_dequantize_fp8 (receiver, in expert order): for every row p of the
 *   dispatch layout, x_perm[p,i] = bf16(code * s + z) of token src_of[p] / k
 *   (float32 multiply and add, bf16 round to nearest even).
 *   codes, scale_zero as written by moe_quantize_fp8; src_of [T*k] from
 *   moe_permute (a value outside [0, T*k) is clamped to a valid token);
 *   x_perm [T*k, d] bf16 out, then the grouped FFN as usual.
 * |x - x_perm| <= (max - min) / 32 per token, plus the bf16 rounding.
 * Returns MOE_EUNSUPPORTED unless dtype is MOE_BF16 and d <= 8192.
 */
int moe_quantize_fp8(const moe_config* cfg, const void* x, uint8_t* codes, float* scale_zero,
                     void* stream);
int moe_dequantize_fp8(const moe_config* cfg, const uint8_t* codes, const int32_t* src_of,
                       const float* scale_zero, void* x_perm, void* stream);

/*
 * moe_ffn_gate_up_packed with the dispatch gather fused into the first GEMM's
 * operand load ([V4-overlap] Waved-EP section: the gather folded into the
 * expert GEMM): row p of expert e's range reads token row x[src_of[p] / k]
 * instead of x_perm[p], so x_perm is never written or read.  Same h, bit for
 * bit, as moe_ffn_gate_up_packed on the x_perm that moe_permute would write.
 *   x       [T, d] bf16 in (16-byte aligned), token order.
 *   src_of  [T*k] int32 in, from moe_permute (values outside [0, T*k) are
 *           clamped to a valid token row, never read out of bounds).
 * The sub-table rule applies: expert_offsets and packed_gate_up may be offset
 * to one rank's experts; src_of stays the whole table.
 */
int moe_ffn_gate_up_packed_gather(const moe_config* cfg, const void* x, const int32_t* src_of,
                                  const int32_t* expert_offsets, const void* packed_gate_up,
                                  void* h, void* stream);

/*
 * ------------------------------------------------------ FP8 first GEMM
 * The first GEMM consuming the per-token FP8 dispatch payload
 * (moe_quantize_fp8: codes c[t, k], (s_t, z_t)) directly, against expert
 * weights quantised once to E4M3 with one scale per output feature
 * ([SyncTax] §3.1: the dispatch payload travels as per-token FP8; the
 * weights' FP8 form is this library's reading):
 *   x^[t, k] = c[t, k] s_t + z_t,   w^[n, k] = q[n, k] s_n,
 *   s_n = max_k |w[n, k]| / 448 (float32), q = E4M3(w / s_n), nearest-even,
 *   h = SiLU(x^ . w^_gate[n]) * (x^ . w^_up[n])     [T*k, f] bf16 out.
 * The matrix instruction multiplies raw codes with float32 accumulation; the
 * epilogue applies s_t s_n and the centre's term z_t s_n sum_k q[n, k].
 * bf16 problems with d a multiple of 128 (MOE_EUNSUPPORTED otherwise).
 *
 * moe_fp8_weight_bytes: bytes of the FP8 gate/up image.
 * moe_pack_weights_fp8: writes the image from w_gate, w_up [E, f, d] bf16
 *   (16-byte aligned; image 256-byte aligned): codes [E][2 f][d] uint8 (per
 *   group of 16 features its 16 gate rows, then its 16 up rows), the float
 *   scales s_n and the float code sums sum_k q[n, k] (exact, then one
 *   float rounding) of the same rows.  A load-time layout, like
 *   moe_pack_weights.
 * moe_ffn_gate_up_fp8_gather: h row p from token src_of[p] / k's codes
 *   (x_codes [T, d] uint8, 16-byte aligned; scale_zero [T, 2] float, from
 *   moe_quantize_fp8), expert_offsets [E+1] as for the grouped FFN.
 */
int moe_fp8_weight_bytes(const moe_config* cfg, size_t* bytes);
int moe_pack_weights_fp8(const moe_config* cfg, const void* w_gate, const void* w_up,
                         void* image, void* stream);
int moe_ffn_gate_up_fp8_gather(const moe_config* cfg, const uint8_t* x_codes,
                               const float* scale_zero, const int32_t* src_of,
                               const int32_t* expert_offsets, const void* image, void* h,
                               void* stream);

/*
 * moe_layer_fwd_packed: when bufs->x_perm is NULL (or bufs is NULL), the
 * dispatch writes indices only and the first GEMM gathers its rows
 * (moe_ffn_gate_up_packed_gather); a given bufs->x_perm is written as by
 * moe_permute and read by moe_ffn_gate_up_packed.  Both give the same out.
 */
int moe_layer_fwd_packed(const moe_config* cfg, const void* x, const void* w_router,
                         const float* bias, const void* packed_gate_up, const void* packed_down,
                         void* out, const moe_layer_bufs* bufs, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * moe_layer_fwd_packed_waved: moe_layer_fwd_packed with the experts in
 * n_waves waves ([V4-overlap] Waved-EP section: the experts are split into
 * waves; inside a wave dispatch, L1 + Act + L2 and combine run in order, and
 * different waves run side by side).  On one GPU there is no exchange to
 * hide, so what the waves overlap is the GEMMs' ragged last rounds and the
 * combine: after the route and the index-only dispatch on `stream`, wave w
 * (experts [w E / n_waves, (w + 1) E / n_waves), their packed images and
 * offsets taken as a sub-table) runs its gather first GEMM, its second GEMM
 * and the combine of the tokens whose highest-numbered chosen expert is in
 * the wave, on `stream` for even w and `aux_stream` for odd w; before that
 * combine the stream waits for wave w - 1, so every token is combined once,
 * after all of its experts, exactly as moe_combine computes it.  On return
 * `stream` waits for every wave (the call is as asynchronous as the others).
 * Outputs are bit for bit those of moe_layer_fwd_packed.
 * n_waves >= 1 and dividing E (MOE_EINVAL otherwise); bufs->x_perm must be
 * NULL (the waves gather their rows); aux_stream NULL or equal to `stream`
 * runs every wave on `stream`.  ws as for moe_layer_fwd_packed.  The call
 * creates and destroys its n_waves + 1 HIP events.
 */
int moe_layer_fwd_packed_waved(const moe_config* cfg, const void* x, const void* w_router,
                               const float* bias, const void* packed_gate_up,
                               const void* packed_down, void* out, const moe_layer_bufs* bufs,
                               void* ws, size_t ws_bytes, int n_waves, void* stream,
                               void* aux_stream);

/*
 * ---------------------------------------------------------------- backward
 * The layer's backward on the routing of its forward pass: the forward's
 * routing indices (topk_idx, slot_of, src_of, expert_offsets) are reused, not
 * recomputed ([SyncTax] §2.4: the backward retraces the forward's routing
 * from the indices the forward kept); each product C = A B gives dA = dC B^T
 * and dW = A^T dC ([V4-overlap], PP bubble section: dW = x^T dy).  bf16 only
 * (MOE_EUNSUPPORTED otherwise); fp32 accumulation; every output is written
 * in full (weight gradients of experts without rows are zero).  All device
 * pointers, 16-byte aligned; asynchronous on `stream`; errors are reported
 * before anything is enqueued.  A full step is
 *   moe_combine_backward -> moe_ffn_backward -> moe_route_backward ->
 *   moe_unpermute_backward.
 */

/*
 * combine backward: out[t] = sum_j g[t,j] y_perm[slot_of[t*k+j]]  =>
 *   d_y_perm[slot_of[t*k+j]] = bf16(g[t,j] d_out[t])   [T*k, d] bf16 out
 *   d_topk_w[t*k+j] = <d_out[t], y_perm[slot_of[t*k+j]]>  [T, k] fp32 out
 * d_out [T, d] bf16, y_perm [T*k, d] bf16 (the forward's), slot_of [T*k],
 * topk_w [T, k] fp32.
 */
int moe_combine_backward(const moe_config* cfg, const void* d_out, const void* y_perm,
                         const int32_t* slot_of, const float* topk_w, void* d_y_perm,
                         float* d_topk_w, void* stream);

/*
 * grouped SwiGLU FFN backward over the expert row segments of x_perm:
 *   a = x Wg_e^T, u = x Wu_e^T (the training forward's, when a and u are
 *     given, [T*k, f] bf16 each; else recomputed from x_perm),
 *   h = SiLU(a) u, dh = dy Wd_e, da = dh u SiLU'(a), du = dh SiLU(a),
 *   d_x_perm = da Wg_e + du Wu_e          [T*k, d] bf16 out
 *   d_w_gate[e] = da_e^T x_e              [E, f, d] bf16 out
 *   d_w_up[e]   = du_e^T x_e              [E, f, d] bf16 out
 *   d_w_down[e] = dy_e^T h_e              [E, d, f] bf16 out
 * x_perm [T*k, d] bf16 (the forward's dispatched rows), expert_offsets [E+1],
 * weights as in moe_grouped_ffn, d_y_perm [T*k, d] bf16.  a and u are both
 * given or both NULL.  packed_dh / packed_dx (each may be NULL): the images
 * moe_pack_weights_backward wrote from these same weights; dh and d_x_perm
 * are then computed on them by the packed kernel (same float32 sums over k
 * in the same order, so the same results within accumulation rounding).
 * ws: moe_workspace_bytes(MOE_ENTRY_FFN_BACKWARD) = 5 T k f bf16 (a, u,
 * dh then h, and da | du side by side per row), 256-byte aligned.
 */
int moe_ffn_backward(const moe_config* cfg, const void* x_perm, const int32_t* expert_offsets,
                     const void* w_gate, const void* w_up, const void* w_down, const void* a,
                     const void* u, const void* packed_dh, const void* packed_dx,
                     const void* d_y_perm, void* d_x_perm, void* d_w_gate, void* d_w_up,
                     void* d_w_down, void* ws, size_t ws_bytes, void* stream);

/*
 * Packed images for the two activation-gradient products of the FFN
 * backward: dh = dy Wd_e needs W_d^T ([E, f, d] view of w_down [E, d, f]),
 * d_x_perm = [da du] [Wg_e; Wu_e] needs [W_g; W_u]^T ([E, d, 2 f] view).
 * Both are written in the plain (down-projection) layout of
 * moe_pack_weights, so the same packed kernel serves them.  Like the
 * forward's images they are a load-time layout: after a weight update they
 * must be written again.
 * moe_packed_weight_bytes_backward: bytes of the two images (bf16 only).
 * moe_pack_weights_backward: writes packed_dh from w_down and/or packed_dx
 *   from w_gate and w_up; either output may be NULL.  Outputs 16-byte
 *   aligned; enqueue-only.
 */
int moe_packed_weight_bytes_backward(const moe_config* cfg, size_t* dh_bytes, size_t* dx_bytes);
int moe_pack_weights_backward(const moe_config* cfg, const void* w_gate, const void* w_up,
                              const void* w_down, void* packed_dh, void* packed_dx,
                              void* stream);

/*
 * Training forward of the first FFN GEMM: moe_ffn_gate_up_packed (src_of ==
 * NULL: act is x_perm) or moe_ffn_gate_up_packed_gather (src_of != NULL: act
 * is the token-order x), which also writes the pre-activations a = x Wg^T and
 * u = x Wu^T ([T*k, f] bf16 each, rounded once from the same fp32 sums as h)
 * for moe_ffn_backward, so the backward does not recompute them.
 */
int moe_ffn_gate_up_packed_train(const moe_config* cfg, const void* act, const int32_t* src_of,
                                 const int32_t* expert_offsets, const void* packed_gate_up,
                                 void* h, void* a, void* u, void* stream);

/*
 * router backward through the gate softmax, selection held fixed:
 *   s = logits + bias; the support set S is the k chosen (renorm), else the
 *   presel pre-selected by (s desc, e asc), else all E; q = softmax of s
 *   over S; dq_e = d_topk_w[t, j] for e = topk_idx[t, j], else 0;
 *   d_logits[t, e] = q_e (dq_e - sum_e' q_e' dq_e') on S, 0 off S  [T, E] fp32 out
 *   d_x_router = dz Wr                     [T, d] bf16 out
 *   d_w_router = dz^T x                    [E, d] bf16 out
 *   d_bias[e] = sum_t dz[t, e] (fixed order; NULL skips)   [E] fp32 out
 * The two products take dz rounded to bf16.  x [T, d] bf16, w_router [E, d]
 * bf16, logits [T, E] fp32 (moe_route's output), bias [E] fp32 or NULL,
 * topk_idx [T, k], d_topk_w [T, k] fp32.  Needs E % 8 == 0; pre-selection
 * without renormalisation together with group-limited routing is
 * MOE_EUNSUPPORTED.  ws: moe_workspace_bytes(MOE_ENTRY_ROUTE_BACKWARD).
 */
int moe_route_backward(const moe_config* cfg, const void* x, const void* w_router,
                       const float* logits, const float* bias, const int32_t* topk_idx,
                       const float* d_topk_w, float* d_logits, void* d_x_router,
                       void* d_w_router, float* d_bias, void* ws, size_t ws_bytes,
                       void* stream);

/*
 * dispatch backward: d_x[t] = sum_j d_x_perm[slot_of[t*k+j]] (+ d_x_router[t]
 * when not NULL), fp32 in j order, then one bf16 rounding.  [T, d] bf16 out.
 */
int moe_unpermute_backward(const moe_config* cfg, const void* d_x_perm, const int32_t* slot_of,
                           const void* d_x_router, void* d_x, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
