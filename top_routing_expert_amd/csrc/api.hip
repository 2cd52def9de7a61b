// C ABI of libmoe_mi355x.so (declared in include/moe.h): host-side argument
// checks, workspace layout and the launch sequence of each entry point.
// Nothing here allocates, frees or synchronises; every check runs before the
// first launch, so a rejected call writes no output.
#include <vector>

#include "common.h"

using namespace moe;

namespace {

constexpr long kI32Max = 2147483647l;

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t elem_bytes(const moe_config& c) { return c.dtype == MOE_BF16 ? 2 : 4; }

// Fields every entry point uses: sizes and element type.
int check_core(const moe_config* c) {
  if (!c) return MOE_EINVAL;
  if (c->T < 0 || c->d <= 0 || c->E <= 0 || c->k <= 0 || c->f <= 0) return MOE_EINVAL;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_EINVAL;
  if (c->k > c->E) return MOE_EINVAL;
  if (c->k > 16 || c->E > kMaxExperts) return MOE_EUNSUPPORTED;
  if (c->dtype == MOE_BF16 && (c->d % 64 || c->f % 64)) return MOE_EUNSUPPORTED;
  if (c->dtype == MOE_F32 && (c->d % 4 || c->f % 4)) return MOE_EUNSUPPORTED;
  const long rows = (long)c->T * c->k;  // < 2^35 (k <= 16)
  const long wide = c->d > c->f ? c->d : c->f;
  // rows * wide > kI32Max, without forming the product (it can pass 2^63)
  if ((rows > 0 && wide > kI32Max / rows) || (long)c->T * c->E > kI32Max)
    return MOE_EUNSUPPORTED;
  return MOE_OK;
}

// Routing fields (router, permute, whole layer).
int check_routing(const moe_config* c) {
  int s = check_core(c);
  if (s != MOE_OK) return s;
  if (c->presel != 0 && (c->presel < c->k || c->presel > c->E)) return MOE_EINVAL;
  if (c->presel > 32) return MOE_EUNSUPPORTED;
  if (c->n_group < 1 || c->E % c->n_group != 0) return MOE_EINVAL;
  if (c->topk_group < 1 || c->topk_group > c->n_group) return MOE_EINVAL;
  if (c->n_group > 64) return MOE_EUNSUPPORTED;
  const int nsel = c->presel > c->k ? c->presel : c->k;
  if ((long)c->topk_group * (c->E / c->n_group) < nsel) return MOE_EINVAL;
  if (c->renorm != 0 && c->renorm != 1) return MOE_EINVAL;
  if (c->ep_ranks < 1 || c->E % c->ep_ranks != 0) return MOE_EINVAL;
  return MOE_OK;
}

size_t route_ws(const moe_config& c) {
  const int s = router_splits(c);
  return s > 1 ? align256((size_t)s * c.T * c.E * sizeof(float)) : 0;
}

// moe_layer_fwd workspace: the route/permute scratch (never live at the same
// time, so they share one region) followed by every intermediate that `bufs`
// does not provide.
struct LayerLayout {
  size_t scratch, logits, idx, w, offs, roffs, slot, src, xperm, h, y, total;
};

LayerLayout layer_layout(const moe_config& c, const moe_layer_bufs* b) {
  LayerLayout L{};
  const size_t A = (size_t)c.T * c.k, es = elem_bytes(c);
  size_t off = 0;
  auto take = [&](size_t bytes, bool provided) {
    const size_t at = off;
    if (!provided) off += align256(bytes);
    return at;
  };
  const size_t rs = route_ws(c), ps = permute_ws_bytes(c);
  L.scratch = take(rs > ps ? rs : ps, false);
  L.logits = take((size_t)c.T * c.E * 4, b && b->logits);
  L.idx = take(A * 4, b && b->topk_idx);
  L.w = take(A * 4, b && b->topk_w);
  L.offs = take(((size_t)c.E + 1) * 4, b && b->expert_offsets);
  L.roffs = take(((size_t)c.ep_ranks + 1) * 4, b && b->rank_offsets);
  L.slot = take(A * 4, b && b->slot_of);
  L.src = take(A * 4, b && b->src_of);
  L.xperm = take(A * c.d * es, b && b->x_perm);
  L.h = take(A * c.f * es, b && b->h);
  L.y = take(A * c.d * es, b && b->y_perm);
  L.total = off;
  return L;
}

int status_of(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

int check_ws(size_t need, const void* ws, size_t ws_bytes) {
  if (need == 0) return MOE_OK;
  if (!ws || ws_bytes < need) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(ws) % 256) return MOE_EINVAL;
  return MOE_OK;
}

// Enqueue-only bodies, called after every check passed.
int do_route(const moe_config& c, const void* x, const void* wr, const float* bias, float* logits,
             int32_t* idx, float* w, void* ws, hipStream_t st) {
  if (c.T == 0) return MOE_OK;
  if (x) {
    if (c.dtype == MOE_F32) {
      hipError_t e = launch_router_gemm_f32(static_cast<const float*>(x),
                                            static_cast<const float*>(wr), logits, c.T, c.d, c.E, st);
      if (e != hipSuccess) return MOE_EHIP;
      return status_of(launch_topk(c, logits, 1, bias, nullptr, idx, w, st));
    }
    const int s = router_splits(c);
    float* dst = s > 1 ? static_cast<float*>(ws) : logits;
    hipError_t e = launch_router_gemm_bf16(static_cast<const uint16_t*>(x),
                                           static_cast<const uint16_t*>(wr), dst, c.T, c.d, c.E, s,
                                           st);
    if (e != hipSuccess) return MOE_EHIP;
    return status_of(launch_topk(c, dst, s, bias, s > 1 ? logits : nullptr, idx, w, st));
  }
  return status_of(launch_topk(c, logits, 1, bias, nullptr, idx, w, st));
}

int do_permute(const moe_config& c, const void* x, const int32_t* idx, int32_t* offs,
               int32_t* roffs, int32_t* slot, int32_t* src, void* xperm, void* ws, hipStream_t st) {
  if (c.T == 0) {
    hipError_t e = launch_fill_i32(offs, c.E + 1, 0, st);
    if (e != hipSuccess) return MOE_EHIP;
    return status_of(launch_fill_i32(roffs, c.ep_ranks + 1, 0, st));
  }
  return status_of(launch_permute(c, x, idx, offs, roffs, slot, src, xperm, ws, st));
}

int do_ffn(const moe_config& c, const void* xperm, const int32_t* offs, const void* wg,
           const void* wu, const void* wd, void* h, void* y, hipStream_t st) {
  if (c.T == 0) return MOE_OK;
  if (wg) {
    hipError_t e = launch_ffn_gate_up(c, xperm, offs, wg, wu, h, st);
    if (e != hipSuccess) return MOE_EHIP;
  }
  if (wd) return status_of(launch_ffn_down(c, h, offs, wd, y, st));
  return MOE_OK;
}

// src non-NULL: `act` is x in token order and the first GEMM gathers its rows.
int do_ffn_packed(const moe_config& c, const void* act, const int32_t* src, const int32_t* offs,
                  const void* pgu, const void* pd, void* h, void* y, hipStream_t st) {
  if (c.T == 0) return MOE_OK;
  if (pgu) {
    hipError_t e = src ? launch_ffn_gate_up_packed_gather(c, act, src, offs, pgu, h, st)
                       : launch_ffn_gate_up_packed(c, act, offs, pgu, h, st);
    if (e != hipSuccess) return MOE_EHIP;
  }
  if (pd) return status_of(launch_ffn_down_packed(c, h, offs, pd, y, st));
  return MOE_OK;
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// Packed-weight entry points: bf16 only, 16-byte aligned operands.
int check_packed(const moe_config* c) {
  int s = check_core(c);
  if (s != MOE_OK) return s;
  if (c->dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

size_t packed_bytes(const moe_config& c, bool gate_up) {
  const PackGeom g = gate_up ? pack_geom(c.f, c.d, true) : pack_geom(c.d, c.f, false);
  return (size_t)c.E * g.expert_elems * 2;
}

int do_combine(const moe_config& c, const void* y, const int32_t* slot, const float* w, void* out,
               hipStream_t st) {
  if (c.T == 0) return MOE_OK;
  return status_of(launch_combine(c, y, slot, w, out, st));
}

// The intermediates of one layer call: the caller's buffers where given,
// else slices of ws.
struct LayerPtrs {
  float* logits;
  int32_t *idx, *offs, *roffs, *slot, *src;
  float* w;
  void *xperm, *h, *y;
  bool gather;  // the first GEMM gathers its rows (no x_perm is written)
};

// Route and dispatch of moe_layer_fwd / moe_layer_fwd_packed(_waved), after
// every argument check passed: with `gather` and no caller x_perm the
// dispatch writes indices only.
int layer_front(const moe_config& c, const void* x, const void* w_router, const float* bias,
                const moe_layer_bufs* bufs, void* ws, size_t ws_bytes, hipStream_t st,
                bool gather, LayerPtrs* P) {
  const LayerLayout L = layer_layout(c, bufs);
  int s;
  if ((s = check_ws(L.total, ws, ws_bytes)) != MOE_OK) return s;
  char* base = static_cast<char*>(ws);
  auto pick = [&](void* given, size_t at) -> void* { return given ? given : base + at; };
  const moe_layer_bufs none{};
  const moe_layer_bufs& b = bufs ? *bufs : none;
  void* scratch = base + L.scratch;
  P->logits = static_cast<float*>(pick(b.logits, L.logits));
  P->idx = static_cast<int32_t*>(pick(b.topk_idx, L.idx));
  P->w = static_cast<float*>(pick(b.topk_w, L.w));
  P->offs = static_cast<int32_t*>(pick(b.expert_offsets, L.offs));
  P->roffs = static_cast<int32_t*>(pick(b.rank_offsets, L.roffs));
  P->slot = static_cast<int32_t*>(pick(b.slot_of, L.slot));
  P->src = static_cast<int32_t*>(pick(b.src_of, L.src));
  P->xperm = pick(b.x_perm, L.xperm);
  P->h = pick(b.h, L.h);
  P->y = pick(b.y_perm, L.y);
  P->gather = gather && !b.x_perm;
  if ((s = do_route(c, x, w_router, bias, P->logits, P->idx, P->w, scratch, st)) != MOE_OK)
    return s;
  return do_permute(c, P->gather ? nullptr : x, P->idx, P->offs, P->roffs, P->slot, P->src,
                    P->gather ? nullptr : P->xperm, scratch, st);
}

// moe_layer_fwd body shared by the row-major and packed-weight variants;
// `ffn(act, src, offs, h, y, stream)` runs the grouped FFN on act = x_perm
// (src NULL) or, with `gather` and no caller x_perm, on act = x with the rows
// gathered through src = src_of.  Routing checks and the FFN's own argument
// checks have passed.
template <typename Ffn>
int run_layer(const moe_config& c, const void* x, const void* w_router, const float* bias,
              void* out, const moe_layer_bufs* bufs, void* ws, size_t ws_bytes, void* stream,
              bool gather, Ffn&& ffn) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  LayerPtrs P;
  int s;
  if ((s = layer_front(c, x, w_router, bias, bufs, ws, ws_bytes, st, gather, &P)) != MOE_OK)
    return s;
  if ((s = ffn(P.gather ? x : P.xperm, P.gather ? P.src : nullptr, P.offs, P.h, P.y, st)) !=
      MOE_OK)
    return s;
  return do_combine(c, P.y, P.slot, P.w, out, st);
}

// Events of one waved call, destroyed on every path out.
struct EventSet {
  std::vector<hipEvent_t> ev;
  ~EventSet() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);  // released once their waits are done
  }
  bool make(int n) {
    for (int i = 0; i < n; ++i) {
      hipEvent_t e;
      if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return false;
      ev.push_back(e);
    }
    return true;
  }
};

// Expert waves after the dispatch: wave w = experts [w per, (w + 1) per) runs
// its first GEMM (rows gathered), its second GEMM and then the combine of the
// tokens whose highest-numbered expert is in the wave, on stream ss[w % 2];
// before that combine the stream waits for wave w - 1 (the other stream), so
// every token is combined once, after all of its experts, exactly as the
// serial combine computes it.  The caller's stream waits for the last wave.
int run_waves(const moe_config& c, const void* x, const LayerPtrs& P, const void* pgu,
              const void* pd, void* out, int n_waves, hipStream_t st, hipStream_t aux) {
  if (c.T == 0) return MOE_OK;
  const int per = c.E / n_waves;
  const bool two = aux && aux != st;
  hipStream_t ss[2] = {st, two ? aux : st};
  EventSet E;
  if (!E.make(n_waves + 1)) return MOE_EHIP;
  hipEvent_t dispatched = E.ev[n_waves];
  if (two && (hipEventRecord(dispatched, st) != hipSuccess ||
              hipStreamWaitEvent(aux, dispatched, 0) != hipSuccess))
    return MOE_EHIP;
  const size_t gu_e = packed_bytes(c, true) / c.E, dn_e = packed_bytes(c, false) / c.E;
  moe_config sub = c;
  sub.E = per;
  for (int w = 0; w < n_waves; ++w) {
    hipStream_t s = ss[w & 1];
    const int32_t* offs_w = P.offs + (size_t)w * per;
    const char* pgu_w = static_cast<const char*>(pgu) + (size_t)w * per * gu_e;
    const char* pd_w = static_cast<const char*>(pd) + (size_t)w * per * dn_e;
    if (launch_ffn_gate_up_packed_gather(sub, x, P.src, offs_w, pgu_w, P.h, s) != hipSuccess ||
        launch_ffn_down_packed(sub, P.h, offs_w, pd_w, P.y, s) != hipSuccess)
      return MOE_EHIP;
    if (two && w > 0 && hipStreamWaitEvent(s, E.ev[w - 1], 0) != hipSuccess) return MOE_EHIP;
    if (launch_combine(c, P.y, P.slot, P.w, out, s, P.idx, w, per) != hipSuccess) return MOE_EHIP;
    if (hipEventRecord(E.ev[w], s) != hipSuccess) return MOE_EHIP;
  }
  if (two && hipStreamWaitEvent(st, E.ev[n_waves - 1], 0) != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (shape, flag, pointer or workspace)";
    case MOE_EUNSUPPORTED: return "valid problem outside what the kernels implement";
    case MOE_EHIP: return "HIP launch failed";
    case MOE_ESCRATCH:
      return "problem needs more scratch than the library's static scratch array holds "
             "(moe_noalloc_scratch_bytes); use the entry point with a workspace";
    default: return "unknown status";
  }
}

int moe_validate(const moe_config* cfg) { return check_routing(cfg); }

int moe_workspace_bytes(const moe_config* cfg, int entry, size_t* bytes) {
  if (!bytes) return MOE_EINVAL;
  int s;
  switch (entry) {
    case MOE_ENTRY_ROUTE:
      if ((s = check_routing(cfg)) != MOE_OK) return s;
      *bytes = route_ws(*cfg);
      return MOE_OK;
    case MOE_ENTRY_PERMUTE:
      if ((s = check_routing(cfg)) != MOE_OK) return s;
      *bytes = cfg->T ? align256(permute_ws_bytes(*cfg)) : 0;
      return MOE_OK;
    case MOE_ENTRY_FFN:
    case MOE_ENTRY_COMBINE:
      if ((s = check_core(cfg)) != MOE_OK) return s;
      *bytes = 0;
      return MOE_OK;
    case MOE_ENTRY_LAYER:
      if ((s = check_routing(cfg)) != MOE_OK) return s;
      *bytes = layer_layout(*cfg, nullptr).total;
      return MOE_OK;
    case MOE_ENTRY_ROUTE_STATS:
      if ((s = check_routing(cfg)) != MOE_OK) return s;
      *bytes = cfg->T ? align256(route_stats_ws_bytes(*cfg)) : 0;
      return MOE_OK;
    case MOE_ENTRY_FFN_BACKWARD:
      if ((s = check_core(cfg)) != MOE_OK) return s;
      *bytes = align256(ffn_backward_ws_bytes(*cfg));
      return MOE_OK;
    case MOE_ENTRY_ROUTE_BACKWARD:
      if ((s = check_routing(cfg)) != MOE_OK) return s;
      *bytes = align256(route_backward_ws_bytes(*cfg));
      return MOE_OK;
    default:
      return MOE_EINVAL;
  }
}

int moe_route(const moe_config* cfg, const void* x, const void* w_router, const float* bias,
              float* logits, int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
              void* stream) {
  int s = check_routing(cfg);
  if (s != MOE_OK) return s;
  const moe_config& c = *cfg;
  if (c.T > 0) {
    if (!logits || !topk_idx || !topk_w) return MOE_EINVAL;
    if (x && !w_router) return MOE_EINVAL;
    if (x && (s = check_ws(route_ws(c), ws, ws_bytes)) != MOE_OK) return s;
  }
  return do_route(c, x, w_router, bias, logits, topk_idx, topk_w, ws,
                  static_cast<hipStream_t>(stream));
}

int moe_permute(const moe_config* cfg, const void* x, const int32_t* topk_idx,
                int32_t* expert_offsets, int32_t* rank_offsets, int32_t* slot_of, int32_t* src_of,
                void* x_perm, void* ws, size_t ws_bytes, void* stream) {
  int s = check_routing(cfg);
  if (s != MOE_OK) return s;
  const moe_config& c = *cfg;
  if (!expert_offsets || !rank_offsets) return MOE_EINVAL;
  if (c.T > 0) {
    // x and x_perm both NULL: index outputs only
    if (!topk_idx || !slot_of || !src_of || (!x != !x_perm)) return MOE_EINVAL;
    if ((s = check_ws(permute_ws_bytes(c), ws, ws_bytes)) != MOE_OK) return s;
  }
  return do_permute(c, x, topk_idx, expert_offsets, rank_offsets, slot_of, src_of, x_perm, ws,
                    static_cast<hipStream_t>(stream));
}

int moe_permute_noalloc(const moe_config* cfg, const void* x, const int32_t* topk_idx,
                        int32_t* expert_offsets, int32_t* rank_offsets, int32_t* slot_of,
                        int32_t* src_of, void* x_perm, void* stream) {
  int s = check_routing(cfg);
  if (s != MOE_OK) return s;
  const moe_config& c = *cfg;
  if (!expert_offsets || !rank_offsets) return MOE_EINVAL;
  void* scratch_ptr = nullptr;
  if (c.T > 0) {
    if (!topk_idx || !slot_of || !src_of || (!x != !x_perm)) return MOE_EINVAL;
    if (permute_ws_bytes(c) > kNoAllocScratchBytes) return MOE_ESCRATCH;
    if (noalloc_scratch(&scratch_ptr) != hipSuccess) return MOE_EHIP;
  }
  return do_permute(c, x, topk_idx, expert_offsets, rank_offsets, slot_of, src_of, x_perm,
                    scratch_ptr, static_cast<hipStream_t>(stream));
}

size_t moe_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

int moe_ffn_gate_up(const moe_config* cfg, const void* x_perm, const int32_t* expert_offsets,
                    const void* w_gate, const void* w_up, void* h, void* stream) {
  int s = check_core(cfg);
  if (s != MOE_OK) return s;
  if (cfg->T > 0 && (!x_perm || !expert_offsets || !w_gate || !w_up || !h)) return MOE_EINVAL;
  return do_ffn(*cfg, x_perm, expert_offsets, w_gate, w_up, nullptr, h, nullptr,
                static_cast<hipStream_t>(stream));
}

int moe_ffn_down(const moe_config* cfg, const void* h, const int32_t* expert_offsets,
                 const void* w_down, void* y_perm, void* stream) {
  int s = check_core(cfg);
  if (s != MOE_OK) return s;
  if (cfg->T > 0 && (!h || !expert_offsets || !w_down || !y_perm)) return MOE_EINVAL;
  return do_ffn(*cfg, nullptr, expert_offsets, nullptr, nullptr, w_down, const_cast<void*>(h),
                y_perm, static_cast<hipStream_t>(stream));
}

int moe_grouped_ffn(const moe_config* cfg, const void* x_perm, const int32_t* expert_offsets,
                    const void* w_gate, const void* w_up, const void* w_down, void* h, void* y_perm,
                    void* stream) {
  int s = check_core(cfg);
  if (s != MOE_OK) return s;
  if (cfg->T > 0 &&
      (!x_perm || !expert_offsets || !w_gate || !w_up || !w_down || !h || !y_perm))
    return MOE_EINVAL;
  return do_ffn(*cfg, x_perm, expert_offsets, w_gate, w_up, w_down, h, y_perm,
                static_cast<hipStream_t>(stream));
}

int moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* slot_of,
                const float* topk_w, void* out, void* stream) {
  int s = check_core(cfg);
  if (s != MOE_OK) return s;
  if (cfg->T > 0 && (!y_perm || !slot_of || !topk_w || !out)) return MOE_EINVAL;
  return do_combine(*cfg, y_perm, slot_of, topk_w, out, static_cast<hipStream_t>(stream));
}

int moe_layer_fwd(const moe_config* cfg, const void* x, const void* w_router, const float* bias,
                  const void* w_gate, const void* w_up, const void* w_down, void* out,
                  const moe_layer_bufs* bufs, void* ws, size_t ws_bytes, void* stream) {
  int s = check_routing(cfg);
  if (s != MOE_OK) return s;
  if (cfg->T > 0 && (!x || !w_router || !w_gate || !w_up || !w_down || !out)) return MOE_EINVAL;
  return run_layer(*cfg, x, w_router, bias, out, bufs, ws, ws_bytes, stream, /*gather=*/false,
                   [&](const void* xp, const int32_t*, const int32_t* offs, void* h, void* y,
                       hipStream_t st) {
                     return do_ffn(*cfg, xp, offs, w_gate, w_up, w_down, h, y, st);
                   });
}

int moe_packed_weight_bytes(const moe_config* cfg, size_t* gate_up_bytes, size_t* down_bytes) {
  int s = check_packed(cfg);
  if (s != MOE_OK) return s;
  if (!gate_up_bytes || !down_bytes) return MOE_EINVAL;
  *gate_up_bytes = packed_bytes(*cfg, true);
  *down_bytes = packed_bytes(*cfg, false);
  return MOE_OK;
}

int moe_pack_weights(const moe_config* cfg, const void* w_gate, const void* w_up,
                     const void* w_down, void* packed_gate_up, void* packed_down, void* stream) {
  int s = check_packed(cfg);
  if (s != MOE_OK) return s;
  if (!packed_gate_up && !packed_down) return MOE_EINVAL;
  if (packed_gate_up && (!w_gate || !w_up || !aligned16(w_gate) || !aligned16(w_up) ||
                         !aligned16(packed_gate_up)))
    return MOE_EINVAL;
  if (packed_down && (!w_down || !aligned16(w_down) || !aligned16(packed_down))) return MOE_EINVAL;
  return status_of(launch_pack_weights(*cfg, w_gate, w_up, w_down, packed_gate_up, packed_down,
                                       static_cast<hipStream_t>(stream)));
}

int moe_packed_weight_bytes_backward(const moe_config* cfg, size_t* dh_bytes, size_t* dx_bytes) {
  int s = check_packed(cfg);
  if (s != MOE_OK) return s;
  if (!dh_bytes || !dx_bytes) return MOE_EINVAL;
  *dh_bytes = (size_t)cfg->E * pack_geom(cfg->f, cfg->d, false).expert_elems * 2;
  *dx_bytes = (size_t)cfg->E * pack_geom(cfg->d, 2 * cfg->f, false).expert_elems * 2;
  return MOE_OK;
}

int moe_pack_weights_backward(const moe_config* cfg, const void* w_gate, const void* w_up,
                              const void* w_down, void* packed_dh, void* packed_dx,
                              void* stream) {
  int s = check_packed(cfg);
  if (s != MOE_OK) return s;
  if (!packed_dh && !packed_dx) return MOE_EINVAL;
  if (packed_dh && (!w_down || !aligned16(packed_dh))) return MOE_EINVAL;
  if (packed_dx && (!w_gate || !w_up || !aligned16(packed_dx))) return MOE_EINVAL;
  return status_of(launch_pack_weights_t(*cfg, w_gate, w_up, w_down, packed_dh, packed_dx,
                                         static_cast<hipStream_t>(stream)));
}

int moe_ffn_gate_up_packed(const moe_config* cfg, const void* x_perm,
                           const int32_t* expert_offsets, const void* packed_gate_up, void* h,
                           void* stream) {
  int s = check_packed(cfg);
  if (s != MOE_OK) return s;
  if (cfg->T > 0 && (!x_perm || !expert_offsets || !packed_gate_up || !h || !aligned16(x_perm) ||
                     !aligned16(packed_gate_up) || !aligned16(h)))
    return MOE_EINVAL;
  return do_ffn_packed(*cfg, x_perm, nullptr, expert_offsets, packed_gate_up, nullptr, h,
                       nullptr, static_cast<hipStream_t>(stream));
}

int moe_route_stats(const moe_config* cfg, const float* logits, const float* bias,
                    const int32_t* expert_offsets, const int32_t* rank_offsets, int32_t* hist,
                    int32_t* rank_load, float* stats, void* ws, size_t ws_bytes, void* stream) {
  int s = check_routing(cfg);
  if (s != MOE_OK) return s;
  if (!hist || !rank_load || !stats) return MOE_EINVAL;
  if (cfg->T > 0) {
    if (!logits || !expert_offsets || !rank_offsets) return MOE_EINVAL;
    if ((s = check_ws(route_stats_ws_bytes(*cfg), ws, ws_bytes)) != MOE_OK) return s;
  }
  return status_of(launch_route_stats(*cfg, logits, bias, expert_offsets, rank_offsets, hist,
                                      rank_load, stats, ws, static_cast<hipStream_t>(stream)));
}

int moe_quantize_fp8(const moe_config* cfg, const void* x, uint8_t* codes, float* scale_zero,
                     void* stream) {
  int s = check_core(cfg);
  if (s != MOE_OK) return s;
  if (!fp8_row_supported(*cfg)) return MOE_EUNSUPPORTED;
  if (cfg->T == 0) return MOE_OK;
  if (!x || !codes || !scale_zero || !aligned16(x) || !aligned16(codes)) return MOE_EINVAL;
  return status_of(launch_fp8_quantize(*cfg, x, codes, scale_zero, static_cast<hipStream_t>(stream)));
}

int moe_dequantize_fp8(const moe_config* cfg, const uint8_t* codes, const int32_t* src_of,
                       const float* scale_zero, void* x_perm, void* stream) {
  int s = check_core(cfg);
  if (s != MOE_OK) return s;
  if (!fp8_row_supported(*cfg)) return MOE_EUNSUPPORTED;
  if (cfg->T == 0) return MOE_OK;
  if (!codes || !src_of || !scale_zero || !x_perm || !aligned16(codes) || !aligned16(x_perm))
    return MOE_EINVAL;
  return status_of(launch_fp8_dequantize(*cfg, codes, src_of, scale_zero, x_perm,
                                         static_cast<hipStream_t>(stream)));
}

int moe_ffn_gate_up_packed_gather(const moe_config* cfg, const void* x, const int32_t* src_of,
                                  const int32_t* expert_offsets, const void* packed_gate_up,
                                  void* h, void* stream) {
  int s = check_packed(cfg);
  if (s != MOE_OK) return s;
  if (cfg->T > 0 && (!x || !src_of || !expert_offsets || !packed_gate_up || !h ||
                     !aligned16(x) || !aligned16(packed_gate_up) || !aligned16(h)))
    return MOE_EINVAL;
  return do_ffn_packed(*cfg, x, src_of, expert_offsets, packed_gate_up, nullptr, h, nullptr,
                       static_cast<hipStream_t>(stream));
}

// FP8 first GEMM: bf16 problems whose hidden size is a multiple of 128 (the
// kernel's k loop takes two 64-wide FP8 steps at a time) and whose rows fit
// the per-token quantiser.
int check_fp8_gemm(const moe_config* cfg) {
  int s = check_packed(cfg);
  if (s != MOE_OK) return s;
  if (cfg->d % 128 || !fp8_row_supported(*cfg)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

int moe_fp8_weight_bytes(const moe_config* cfg, size_t* bytes) {
  int s = check_fp8_gemm(cfg);
  if (s != MOE_OK) return s;
  if (!bytes) return MOE_EINVAL;
  *bytes = fp8_geom(*cfg).total;
  return MOE_OK;
}

int moe_pack_weights_fp8(const moe_config* cfg, const void* w_gate, const void* w_up,
                         void* image, void* stream) {
  int s = check_fp8_gemm(cfg);
  if (s != MOE_OK) return s;
  if (!w_gate || !w_up || !image || !aligned16(w_gate) || !aligned16(w_up) ||
      reinterpret_cast<uintptr_t>(image) % 256)
    return MOE_EINVAL;
  return status_of(launch_pack_weights_fp8(*cfg, w_gate, w_up, image,
                                           static_cast<hipStream_t>(stream)));
}

int moe_ffn_gate_up_fp8_gather(const moe_config* cfg, const uint8_t* x_codes,
                               const float* scale_zero, const int32_t* src_of,
                               const int32_t* expert_offsets, const void* image, void* h,
                               void* stream) {
  int s = check_fp8_gemm(cfg);
  if (s != MOE_OK) return s;
  if (cfg->T == 0) return MOE_OK;
  if (!x_codes || !scale_zero || !src_of || !expert_offsets || !image || !h ||
      !aligned16(x_codes) || reinterpret_cast<uintptr_t>(scale_zero) % 8 ||
      reinterpret_cast<uintptr_t>(image) % 256 || !aligned16(h))
    return MOE_EINVAL;
  return status_of(launch_ffn_gate_up_fp8_gather(*cfg, x_codes, scale_zero, src_of,
                                                 expert_offsets, image, h,
                                                 static_cast<hipStream_t>(stream)));
}

int moe_ffn_gate_up_packed_train(const moe_config* cfg, const void* act, const int32_t* src_of,
                                 const int32_t* expert_offsets, const void* packed_gate_up,
                                 void* h, void* a, void* u, void* stream) {
  int s = check_packed(cfg);
  if (s != MOE_OK) return s;
  if (cfg->T == 0) return MOE_OK;
  if (!act || !expert_offsets || !packed_gate_up || !h || !a || !u || !aligned16(act) ||
      !aligned16(packed_gate_up) || !aligned16(h) || !aligned16(a) || !aligned16(u))
    return MOE_EINVAL;
  return status_of(launch_ffn_gate_up_packed_save(*cfg, act, src_of, expert_offsets,
                                                  packed_gate_up, h, a, u,
                                                  static_cast<hipStream_t>(stream)));
}

int moe_ffn_down_packed(const moe_config* cfg, const void* h, const int32_t* expert_offsets,
                        const void* packed_down, void* y_perm, void* stream) {
  int s = check_packed(cfg);
  if (s != MOE_OK) return s;
  if (cfg->T > 0 && (!h || !expert_offsets || !packed_down || !y_perm || !aligned16(h) ||
                     !aligned16(packed_down) || !aligned16(y_perm)))
    return MOE_EINVAL;
  return do_ffn_packed(*cfg, nullptr, nullptr, expert_offsets, nullptr, packed_down,
                       const_cast<void*>(h), y_perm, static_cast<hipStream_t>(stream));
}

int moe_layer_fwd_packed(const moe_config* cfg, const void* x, const void* w_router,
                         const float* bias, const void* packed_gate_up, const void* packed_down,
                         void* out, const moe_layer_bufs* bufs, void* ws, size_t ws_bytes,
                         void* stream) {
  int s = check_routing(cfg);
  if (s != MOE_OK) return s;
  if ((s = check_packed(cfg)) != MOE_OK) return s;
  if (cfg->T > 0 && (!x || !w_router || !packed_gate_up || !packed_down || !out || !aligned16(x) ||
                     !aligned16(packed_gate_up) || !aligned16(packed_down)))
    return MOE_EINVAL;
  if (bufs && ((bufs->x_perm && !aligned16(bufs->x_perm)) || (bufs->h && !aligned16(bufs->h)) ||
               (bufs->y_perm && !aligned16(bufs->y_perm))))
    return MOE_EINVAL;
  return run_layer(*cfg, x, w_router, bias, out, bufs, ws, ws_bytes, stream, /*gather=*/true,
                   [&](const void* act, const int32_t* src, const int32_t* offs, void* h, void* y,
                       hipStream_t st) {
                     return do_ffn_packed(*cfg, act, src, offs, packed_gate_up, packed_down, h, y,
                                          st);
                   });
}

int moe_layer_fwd_packed_waved(const moe_config* cfg, const void* x, const void* w_router,
                               const float* bias, const void* packed_gate_up,
                               const void* packed_down, void* out, const moe_layer_bufs* bufs,
                               void* ws, size_t ws_bytes, int n_waves, void* stream,
                               void* aux_stream) {
  int s = check_routing(cfg);
  if (s != MOE_OK) return s;
  if ((s = check_packed(cfg)) != MOE_OK) return s;
  if (n_waves < 1 || cfg->E % n_waves) return MOE_EINVAL;
  if (bufs && bufs->x_perm) return MOE_EINVAL;  // the waves gather their rows
  if (cfg->T > 0 && (!x || !w_router || !packed_gate_up || !packed_down || !out || !aligned16(x) ||
                     !aligned16(packed_gate_up) || !aligned16(packed_down)))
    return MOE_EINVAL;
  if (bufs && ((bufs->h && !aligned16(bufs->h)) || (bufs->y_perm && !aligned16(bufs->y_perm))))
    return MOE_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  LayerPtrs P;
  if ((s = layer_front(*cfg, x, w_router, bias, bufs, ws, ws_bytes, st, /*gather=*/true, &P)) !=
      MOE_OK)
    return s;
  return run_waves(*cfg, x, P, packed_gate_up, packed_down, out, n_waves, st,
                   static_cast<hipStream_t>(aux_stream));
}

int moe_combine_backward(const moe_config* cfg, const void* d_out, const void* y_perm,
                         const int32_t* slot_of, const float* topk_w, void* d_y_perm,
                         float* d_topk_w, void* stream) {
  int s = check_core(cfg);
  if (s != MOE_OK) return s;
  if (cfg->dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (cfg->T == 0) return MOE_OK;
  if (!d_out || !y_perm || !slot_of || !topk_w || !d_y_perm || !d_topk_w || !aligned16(d_out) ||
      !aligned16(y_perm) || !aligned16(d_y_perm))
    return MOE_EINVAL;
  return status_of(launch_combine_backward(*cfg, d_out, y_perm, slot_of, topk_w, d_y_perm,
                                           d_topk_w, static_cast<hipStream_t>(stream)));
}

int moe_ffn_backward(const moe_config* cfg, const void* x_perm, const int32_t* expert_offsets,
                     const void* w_gate, const void* w_up, const void* w_down, const void* a,
                     const void* u, const void* packed_dh, const void* packed_dx,
                     const void* d_y_perm, void* d_x_perm, void* d_w_gate, void* d_w_up,
                     void* d_w_down, void* ws, size_t ws_bytes, void* stream) {
  int s = check_core(cfg);
  if (s != MOE_OK) return s;
  if (cfg->dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (!expert_offsets || !w_gate || !w_up || !w_down || !d_w_gate || !d_w_up || !d_w_down)
    return MOE_EINVAL;
  if (cfg->T > 0 && (!x_perm || !d_y_perm || !d_x_perm)) return MOE_EINVAL;
  if (!a != !u) return MOE_EINVAL;
  const void* al[] = {x_perm, w_gate, w_up, w_down, a, u, packed_dh, packed_dx, d_y_perm,
                      d_x_perm, d_w_gate, d_w_up, d_w_down, ws};
  for (const void* p : al)
    if (p && !aligned16(p)) return MOE_EINVAL;
  if ((s = check_ws(ffn_backward_ws_bytes(*cfg), ws, ws_bytes)) != MOE_OK) return s;
  return status_of(launch_ffn_backward(*cfg, x_perm, expert_offsets, w_gate, w_up, w_down, a, u,
                                       packed_dh, packed_dx, d_y_perm, d_x_perm, d_w_gate,
                                       d_w_up, d_w_down, ws, static_cast<hipStream_t>(stream)));
}

int moe_route_backward(const moe_config* cfg, const void* x, const void* w_router,
                       const float* logits, const float* bias, const int32_t* topk_idx,
                       const float* d_topk_w, float* d_logits, void* d_x_router,
                       void* d_w_router, float* d_bias, void* ws, size_t ws_bytes,
                       void* stream) {
  int s = check_routing(cfg);
  if (s != MOE_OK) return s;
  const moe_config& c = *cfg;
  if (c.dtype != MOE_BF16 || c.E % 8) return MOE_EUNSUPPORTED;
  if (!c.renorm && c.presel > 0 && c.n_group > 1 && c.topk_group < c.n_group)
    return MOE_EUNSUPPORTED;
  if (!w_router || !d_w_router) return MOE_EINVAL;
  if (c.T > 0 && (!x || !logits || !topk_idx || !d_topk_w || !d_logits || !d_x_router))
    return MOE_EINVAL;
  const void* al[] = {x, w_router, d_x_router, d_w_router, ws};
  for (const void* p : al)
    if (p && !aligned16(p)) return MOE_EINVAL;
  if ((s = check_ws(route_backward_ws_bytes(c), ws, ws_bytes)) != MOE_OK) return s;
  return status_of(launch_route_backward(c, x, w_router, logits, bias, topk_idx, d_topk_w,
                                         d_logits, d_x_router, d_w_router, d_bias, ws,
                                         static_cast<hipStream_t>(stream)));
}

int moe_unpermute_backward(const moe_config* cfg, const void* d_x_perm, const int32_t* slot_of,
                           const void* d_x_router, void* d_x, void* stream) {
  int s = check_core(cfg);
  if (s != MOE_OK) return s;
  if (cfg->dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (cfg->T == 0) return MOE_OK;
  if (!d_x_perm || !slot_of || !d_x || !aligned16(d_x_perm) || !aligned16(d_x) ||
      (d_x_router && !aligned16(d_x_router)))
    return MOE_EINVAL;
  return status_of(launch_unpermute_backward(*cfg, d_x_perm, slot_of, d_x_router, d_x,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"
