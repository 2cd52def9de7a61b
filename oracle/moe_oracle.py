"""CPU oracle of the MoE-layer forward token path and of its backward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only the tests, the package smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library (no kernels,
headers, helpers, tables or pre/post-processing); the only thing both sides
consume is the seeded input generator, which holds none of the method's
arithmetic.

Everything is plain NumPy in float64 (inputs given as bf16 or fp32 are widened
exactly), written step by step in the order the method is stated, with no
blocking, fusion or reordering.  The one deliberate fp32 operation is the
score add s = fp32(z) + fp32(b) (see `scores`), because the routing decision is
defined on fp32 scores and both sides must take it in the same precision.

Pages cited (by title and section):
  [EP-V4]    "DeepSeek-V4的Expert Parallelism与计算通信遮掩实战解析" (tqpw.cn)
  [ThunderEP] ThunderEP article on MoE expert parallelism over PCIe (discosf.com),
             section 2 "MoE专家并行的通信本质"
  [V4-overlap] "DeepSeek-v4 Parallel comp-comm overlap" (recsys-frontier blog),
             sections "先让 EP 在 IB 网络上跑起来" and "V4 的 Waved-EP 通信计算遮掩"
  [SyncTax]  "Deepseek-MoE同步税本质与四层实战优化指南" (qwbw.cn)

Readings taken where the pages are silent or disagree (each is also listed in
the design notes): ties go to the lowest expert / group index; selection is on
fp32 scores, -0 equal to +0; the group score is the max over the group;
groups and expert-to-rank blocks are contiguous; the order inside an expert's
segment is ascending token index; no capacity limit (dropless); SwiGLU is
SiLU(x Wg^T) * (x Wu^T) then W_down; without renormalisation and without
pre-selection the gate denominator runs over all E experts.  The backward
holds the forward's selection fixed (it is piecewise constant), so the router
gets its gradient through the gate weights only; the per-expert bias, added
to the logits before the softmax, gets sum_t dz[t].

Parity pins: every function here is pinned by `-m "not gpu"` tests against
closed forms, hand-worked cases, brute force or library routines; none is
"parity unpinned".
"""
from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np

__all__ = [
    "widen_bf16", "router_logits", "scores", "select", "gates", "margins", "route",
    "permute", "silu", "expert_ffn", "grouped_ffn", "combine", "layer",
    "select_bruteforce", "dense_bruteforce", "combine_backward", "expert_ffn_backward",
    "grouped_ffn_backward", "scatter_rows_backward", "gates_backward", "layer_backward",
    "swiglu_backward", "quantize_weights_fp8", "gate_up_fp8",
]


# ----------------------------------------------------------------------------
# input widening
# ----------------------------------------------------------------------------
def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of fp32)."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("widen_bf16 expects uint16 bit patterns")
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return widen_bf16(a)
    return a.astype(np.float64)


# ----------------------------------------------------------------------------
# a1: router gate GEMM
# ----------------------------------------------------------------------------
def router_logits(x, w_router) -> np.ndarray:
    """z[t, e] = sum_i x[t, i] * Wr[e, i], in float64.

    Every machine computes the gate logits of a token over the experts before
    choosing top-k ([EP-V4] §2.1; [SyncTax] §2.1 gating network).
    """
    return _f64(x) @ _f64(w_router).T


# ----------------------------------------------------------------------------
# a2: scores, selection, gates
# ----------------------------------------------------------------------------
def scores(z32, bias=None) -> np.ndarray:
    """s = fp32(z) + fp32(b) as one IEEE single-precision add, then -0 -> +0.

    The per-expert bias is added to the router logits before selection and
    softmax (the workloads' "router logits given a per-expert bias").  The
    result stays float32: the routing decision is defined on these values.
    """
    s = np.asarray(z32, dtype=np.float32)
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float32)[None, :]
    return s + np.float32(0.0)  # -0.0 + +0.0 = +0.0 under round-to-nearest


def _order_desc(v: np.ndarray) -> np.ndarray:
    """Per row, indices ordered by (value descending, index ascending)."""
    return np.argsort(-v, axis=-1, kind="stable")


def _eligible(s: np.ndarray, n_group: int, topk_group: int) -> np.ndarray:
    """Mask of experts inside the kept groups (group-limited routing).

    Experts form n_group contiguous groups; a group's score is the max of its
    experts' scores; the `topk_group` best groups by (score desc, group asc)
    are kept and all other experts are excluded ([V4-overlap], "先让 EP 在 IB
    网络上跑起来": the 8 experts may only come from the best 4 nodes).
    """
    T, E = s.shape
    if n_group <= 1 or topk_group >= n_group:
        return np.ones((T, E), dtype=bool)
    gs = E // n_group
    group_score = s.reshape(T, n_group, gs).max(axis=2)
    kept = _order_desc(group_score)[:, :topk_group]
    gmask = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(gmask, kept, True, axis=1)
    return np.repeat(gmask, gs, axis=1)


def select(s, k: int, n_group: int = 1, topk_group: int = 1, presel: int = 0) -> np.ndarray:
    """Experts in order (s desc, e asc) among the eligible ones.

    Returns the first max(k, presel) indices per token, best first: the first k
    are the chosen experts, the first `presel` the partial top-P set over which
    the softmax is taken ([EP-V4] §3.2: partial sort to the top-8 logits).
    """
    s = np.asarray(s, dtype=np.float32)
    elig = _eligible(s, n_group, topk_group)
    key = np.where(elig, s.astype(np.float64), -np.inf)
    return _order_desc(key)[:, : max(k, presel)]


def gates(s, sel, k: int, presel: int = 0, renorm: int = 1) -> np.ndarray:
    """Softmax gate weights of the k chosen experts, float64.

    m is the best score (max subtraction before the exponential, [EP-V4] §3.2);
    e_j = exp(s_j - m).  renorm=1: g_j = e_j / sum over the k chosen.
    presel=P, renorm=0: g_j = e_j / sum over the P pre-selected ([EP-V4] §3.2:
    exact softmax over only the top-8, then take the top-2).
    presel=0, renorm=0: the denominator runs over all E experts.
    """
    s64 = np.asarray(s, dtype=np.float32).astype(np.float64)
    top = np.take_along_axis(s64, sel, axis=1)
    m = top[:, :1]
    e = np.exp(top - m)
    if renorm:
        denom = e[:, :k].sum(axis=1)
    elif presel:
        denom = e[:, :presel].sum(axis=1)
    else:
        denom = np.exp(s64 - m).sum(axis=1)
    return e[:, :k] / denom[:, None]


def margins(s64, k: int, n_group: int = 1, topk_group: int = 1) -> np.ndarray:
    """Per token, the smallest gap at a selection boundary, in float64.

    The k-th minus (k+1)-th eligible score, and with group-limited routing also
    the topk_group-th minus (topk_group+1)-th group score.  A token whose gap is
    below the flip threshold may legitimately be routed differently by an fp32
    computation of the logits.
    """
    s64 = np.asarray(s64, dtype=np.float64)
    T, E = s64.shape
    elig = _eligible(s64, n_group, topk_group)
    srt = -np.sort(-np.where(elig, s64, -np.inf), axis=1)
    gap = np.full(T, np.inf)
    if k < E:
        gap = srt[:, k - 1] - srt[:, k]  # finite - (-inf) = +inf when too few are eligible
    if n_group > 1 and topk_group < n_group:
        gsc = -np.sort(-s64.reshape(T, n_group, E // n_group).max(axis=2), axis=1)
        gap = np.minimum(gap, gsc[:, topk_group - 1] - gsc[:, topk_group])
    return gap


def route(logits32, bias, *, k, n_group=1, topk_group=1, presel=0, renorm=1):
    """Scores -> selection -> gates.  Returns (topk_idx int32 [T,k], topk_w f64 [T,k], s f32)."""
    s = scores(logits32, bias)
    sel = select(s, k, n_group, topk_group, presel)
    w = gates(s, sel, k, presel, renorm)
    return sel[:, :k].astype(np.int32), w, s


# ----------------------------------------------------------------------------
# a3 + a4: histogram, offsets, stable permutation (dispatch layout)
# ----------------------------------------------------------------------------
def permute(topk_idx, E: int, ep_ranks: int = 1) -> dict:
    """Expert-contiguous dispatch layout.

    c_e = number of (token, choice) pairs routed to e; o = exclusive prefix sum
    of c (the count identity sum c_e = T*k: [ThunderEP] §2, 1024 tokens with
    top-2 are 2048 expert calls).  The rows of expert e are its tokens in
    ascending token order: p(t, j) = o_e + #{t' < t routed to e}.  Rows are
    packed per destination with one chunk per expert in expert-ID order
    ([EP-V4] §3.3), and experts are placed on ranks in contiguous blocks of
    E/R ([EP-V4] §3.1 example: experts 0-7 on machine 0, 8-15 on machine 1),
    so rank r's send chunk starts at rank_offsets[r] = o[r * E/R].
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = idx.shape
    flat = idx.reshape(-1)  # entry i = t*k + j
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    slot_of = np.empty(T * k, dtype=np.int64)
    for e in range(E):
        # ascending entry index == ascending token, since a token picks e at most once
        entries = np.flatnonzero(flat == e)
        slot_of[entries] = offsets[e] + np.arange(entries.size)
    src_of = np.empty(T * k, dtype=np.int64)
    src_of[slot_of] = np.arange(T * k)
    per_rank = E // ep_ranks
    rank_offsets = offsets[np.arange(ep_ranks + 1) * per_rank]
    return {
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "rank_offsets": rank_offsets.astype(np.int32),
        "slot_of": slot_of.astype(np.int32),
        "src_of": src_of.astype(np.int32),
    }


# ----------------------------------------------------------------------------
# Routing diagnostics (by-products of a2 / a3)
# ----------------------------------------------------------------------------
def route_stats(logits32, bias, topk_idx, E: int, ep_ranks: int = 1, presel: int = 0) -> dict:
    """Load-balance diagnostics of one batch's routing.

    [SyncTax] §5.1 reports the activation frequency of every expert and the
    entropy of the routing as its load-balance measure (ideal log2 E bits:
    4.0 for 16 experts); [EP-V4] §6.2 reports per-expert activation shares
    against the ideal 1/E.  Readings (the pages give no formulas): the
    histogram is the number of (token, choice) pairs per expert (the
    dispatch's c_e); the load entropy is -sum_e q_e log2 q_e over the shares
    q_e = c_e / (T k), terms with q_e = 0 dropped; the maximum load ratio is
    E * max_e c_e / (T k) (1 = perfectly even); the per-rank load sums the
    histogram over each rank's contiguous block of E/R experts.  The token
    entropy is the mean over tokens of -sum_e p_e log2 p_e, p = softmax over
    all E experts of the fp32 scores s = z + b; the pre-selection gap
    (presel P > 0) is the mean over tokens of the softmax mass outside the P
    pre-selected experts (order: s desc, e asc), i.e. what the partial
    softmax over P leaves out.  A batch of no tokens gives zeros.
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    T = idx.shape[0]
    hist = np.bincount(idx.reshape(-1), minlength=E)[:E]
    rank_load = hist.reshape(ep_ranks, E // ep_ranks).sum(axis=1)
    A = idx.size
    load_entropy = max_ratio = token_entropy = gap = 0.0
    if A:
        q = hist / A
        nz = q > 0
        load_entropy = float(-(q[nz] * np.log2(q[nz])).sum())
        max_ratio = float(E * hist.max() / A)
    if T:
        s = scores(logits32, bias).astype(np.float64)
        ex = np.exp(s - s.max(axis=1, keepdims=True))
        p = ex / ex.sum(axis=1, keepdims=True)
        with np.errstate(divide="ignore", invalid="ignore"):
            plogp = np.where(p > 0, p * np.log2(p), 0.0)
        token_entropy = float((-plogp.sum(axis=1)).mean())
        if presel:
            top = _order_desc(s)[:, :presel]
            gap = float((1.0 - np.take_along_axis(p, top, axis=1).sum(axis=1)).mean())
    return {
        "hist": hist.astype(np.int32),
        "rank_load": rank_load.astype(np.int32),
        "token_entropy_bits": token_entropy,
        "presel_gap": gap,
        "load_entropy_bits": load_entropy,
        "max_load_ratio": max_ratio,
    }


# ----------------------------------------------------------------------------
# Per-token FP8 compression of the dispatch payload ([SyncTax] §3.1)
# ----------------------------------------------------------------------------
F8_MAX = 448.0  # largest finite E4M3 value: 1.75 * 2^8


def fp8_e4m3_decode(codes) -> np.ndarray:
    """E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
    infinities, S.1111.111 = NaN) -> float64, exactly."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e4 = (c >> 3) & 0xF
    m3 = c & 0x7
    mag = np.where(e4 == 0, m3 * 2.0 ** -9, (1.0 + m3 / 8.0) * np.exp2(e4 - 7.0))
    return sign * mag


def fp8_e4m3_encode(v) -> np.ndarray:
    """float32 values with |v| <= 448 -> E4M3 codes, rounding to nearest,
    ties to the even code.  Below 2^-6 the step is 2^-9 (subnormals); in the
    binade [2^e, 2^(e+1)) it is 2^(e-3).  Every step is exact in float32."""
    v = np.asarray(v, dtype=np.float32)
    sign = np.signbit(v).astype(np.int64) << 7
    a = np.abs(v).astype(np.float32)
    sub = a < np.float32(2.0 ** -6)
    m_sub = np.rint(a * np.float32(512.0)).astype(np.int64)        # 0 .. 8 (8 = 2^-6)
    f, E = np.frexp(a)                                              # a = f 2^E, f in [0.5, 1)
    e = E.astype(np.int64) - 1
    mant = np.ldexp(f, 1).astype(np.float32)                        # [1, 2)
    m = np.rint((mant - np.float32(1.0)) * np.float32(8.0)).astype(np.int64)
    up = m == 8
    e = np.where(up, e + 1, e)
    m = np.where(up, 0, m)
    normal = ((e + 7) << 3) | m
    return (np.where(sub, m_sub, normal) | sign).astype(np.uint8)


def round_bf16(v32) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite values)."""
    b = np.asarray(v32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def quantize_rows_fp8(x_bits) -> tuple:
    """Per-token affine FP8: each row's [min, max] is mapped onto [-448, 448]
    ([SyncTax] §3.1: every token's vector gets its own min/max and an affine
    map, so one outlier does not widen every token's range).  Readings: the
    centre z = (max + min) / 2 and the scale s = ((max - min) / 2) / 448 are
    float32, v = (x - z) / s in float32 (0 for a constant row, s = 0), clamped
    to +-448 and rounded to E4M3 by fp8_e4m3_encode.  Returns (codes uint8
    [T, d], scale float32 [T], zero float32 [T])."""
    x = widen_bf16(np.asarray(x_bits, dtype=np.uint16)).astype(np.float32)
    hi = x.max(axis=1)
    lo = x.min(axis=1)
    z = ((hi + lo) * np.float32(0.5)).astype(np.float32)
    hr = ((hi - lo) * np.float32(0.5)).astype(np.float32)
    s = (hr / np.float32(F8_MAX)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(s[:, None] > 0, (x - z[:, None]) / s[:, None], np.float32(0.0)).astype(np.float32)
    v = np.clip(v, np.float32(-F8_MAX), np.float32(F8_MAX))
    return fp8_e4m3_encode(v), s, z


def dequantize_rows_fp8(codes, scale, zero) -> np.ndarray:
    """x^ = code * s + z (float32 multiply, then float32 add), rounded to bf16."""
    q = fp8_e4m3_decode(codes).astype(np.float32)
    s = np.asarray(scale, np.float32)[:, None]
    z = np.asarray(zero, np.float32)[:, None]
    return round_bf16(((q * s).astype(np.float32) + z).astype(np.float32))


def quantize_weights_fp8(w):
    """Per-output-channel symmetric FP8 (E4M3) of expert weights [..., F, K]
    (bf16 bit patterns or floats), for an FP8 first GEMM fed by the per-token
    FP8 payload above ([SyncTax] §3.1 sends the dispatch payload in FP8; the
    weights of the GEMM that consumes it are this path's reading).  Readings:
    one scale per output feature n (a weight row), s_n = max_k |w[n, k]| / 448
    in float32, so every row uses the whole E4M3 range and one large row does
    not coarsen the others; weights are centred, so no zero point; v = w / s_n
    in float32 (0 for an all-zero row, s_n = 0), clamped to +-448 and rounded
    by fp8_e4m3_encode.  Returns (codes uint8 [..., F, K], scale float32
    [..., F])."""
    a = np.asarray(w)
    x = (widen_bf16(a) if a.dtype == np.uint16 else a.astype(np.float64)).astype(np.float32)
    m = np.abs(x).max(axis=-1)
    s = (m / np.float32(F8_MAX)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(s[..., None] > 0, x / s[..., None], np.float32(0.0)).astype(np.float32)
    v = np.clip(v, np.float32(-F8_MAX), np.float32(F8_MAX))
    return fp8_e4m3_encode(v), s


def gate_up_fp8(x_codes, x_scale, x_zero, wg_codes, wg_scale, wu_codes, wu_scale):
    """The expert's first GEMM on FP8 operands, exactly: the token rows are
    x^[k] = code * s_t + z_t (the per-token affine payload), the weights
    w^[n, k] = code * s_n (per output feature); a = x^ . w^_g[n],
    u = x^ . w^_u[n] and h = SiLU(a) * u, all in float64 on the decoded
    values with no intermediate rounding.  Returns (h, a, u) [rows, F]."""
    xd = (fp8_e4m3_decode(x_codes) * np.asarray(x_scale, np.float64)[:, None]
          + np.asarray(x_zero, np.float64)[:, None])
    wg = fp8_e4m3_decode(wg_codes) * np.asarray(wg_scale, np.float64)[:, None]
    wu = fp8_e4m3_decode(wu_codes) * np.asarray(wu_scale, np.float64)[:, None]
    a = xd @ wg.T
    u = xd @ wu.T
    return silu(a) * u, a, u


def gather_rows(x, src_of, k: int) -> np.ndarray:
    """x_perm[p] = x[src_of[p] // k]: a plain row copy (bit patterns kept)."""
    return np.asarray(x)[np.asarray(src_of) // k]


# ----------------------------------------------------------------------------
# a5 + a6: per-expert SwiGLU FFN
# ----------------------------------------------------------------------------
def silu(a):
    """SiLU(a) = a * sigmoid(a) = a / (1 + exp(-a))."""
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def expert_ffn(X, w_gate_e, w_up_e, w_down_e):
    """One expert on its rows: h = SiLU(X Wg^T) * (X Wu^T); y = h Wd^T (float64).

    The expert FFN is "L1 + Act + L2" ([V4-overlap], Waved-EP section); the
    gated (SwiGLU) form and the [f,d] / [f,d] / [d,f] per-expert layouts are
    this path's reading.  Returns (y, h).
    """
    X = _f64(X)
    a = X @ _f64(w_gate_e).T
    u = X @ _f64(w_up_e).T
    h = silu(a) * u
    return h @ _f64(w_down_e).T, h


def grouped_ffn(x_perm, offsets, w_gate, w_up, w_down):
    """Run every expert on its segment [o_e, o_{e+1}) of the permuted rows."""
    x_perm = np.asarray(x_perm)
    A = x_perm.shape[0]
    E = len(offsets) - 1
    f = np.asarray(w_gate).shape[1]
    d = np.asarray(w_down).shape[1]
    y = np.zeros((A, d))
    h = np.zeros((A, f))
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            y[r0:r1], h[r0:r1] = expert_ffn(x_perm[r0:r1], w_gate[e], w_up[e], w_down[e])
    return y, h


# ----------------------------------------------------------------------------
# a7: weighted combine
# ----------------------------------------------------------------------------
def combine(y_perm, slot_of, topk_w) -> np.ndarray:
    """out[t] = sum over j ascending of g[t, j] * y[p(t, j)] (float64).

    Each token's k expert outputs are summed with their gate weights back on
    the token's home device ([SyncTax] §2.3).
    """
    g = np.asarray(topk_w, dtype=np.float64)
    T, k = g.shape
    y = _f64(y_perm)
    slots = np.asarray(slot_of).reshape(T, k)
    out = np.zeros((T, y.shape[1]))
    for j in range(k):
        out += g[:, j : j + 1] * y[slots[:, j]]
    return out


# ----------------------------------------------------------------------------
# the whole layer
# ----------------------------------------------------------------------------
def layer(x, w_router, bias, w_gate, w_up, w_down, *, k, n_group=1, topk_group=1,
          presel=0, renorm=1, ep_ranks=1, logits32=None) -> dict:
    """router -> permute -> grouped FFN -> combine, serial as the method states
    ([V4-overlap]: dispatch, expert compute and combine are three serial steps;
    [SyncTax] §2.1-§2.3).

    `logits32` (fp32) replaces the oracle's own logits when given, so that the
    rest of the path can be checked on another implementation's routing inputs.
    """
    E = np.asarray(w_router).shape[0]
    z = router_logits(x, w_router)
    z32 = z.astype(np.float32) if logits32 is None else np.asarray(logits32, np.float32)
    idx, w, s = route(z32, bias, k=k, n_group=n_group, topk_group=topk_group,
                      presel=presel, renorm=renorm)
    s64 = z + (0.0 if bias is None else np.asarray(bias, np.float32).astype(np.float64)[None, :])
    perm = permute(idx, E, ep_ranks)
    x_perm = gather_rows(x, perm["src_of"], k)
    y, h = grouped_ffn(x_perm, perm["offsets"], w_gate, w_up, w_down)
    out = combine(y, perm["slot_of"], w)
    return dict(logits=z, s=s, topk_idx=idx, topk_w=w, margin=margins(s64, k, n_group, topk_group),
                x_perm=x_perm, h=h, y_perm=y, out=out, **perm)


# ----------------------------------------------------------------------------
# layer backward: the mirror of the forward on the cached routing
# ----------------------------------------------------------------------------
def combine_backward(d_out, y_perm, slot_of, topk_w):
    """out[t] = sum_j g[t, j] y[p(t, j)]  =>
    dy[p(t, j)] = g[t, j] d_out[t]  and  dg[t, j] = <d_out[t], y[p(t, j)]>.
    Returns (dy_perm [A, d], dg [T, k]), float64."""
    dout = _f64(d_out)
    g = np.asarray(topk_w, dtype=np.float64)
    T, k = g.shape
    y = _f64(y_perm)
    slots = np.asarray(slot_of).reshape(T, k)
    dy = np.zeros_like(y)
    dg = np.zeros((T, k))
    for j in range(k):
        dy[slots[:, j]] = g[:, j : j + 1] * dout
        dg[:, j] = np.sum(dout * y[slots[:, j]], axis=1)
    return dy, dg


def swiglu_backward(a, u, dh):
    """The activation step of the expert's backward: h = SiLU(a) * u, so a
    gradient dh gives da = dh * u * SiLU'(a) and du = dh * SiLU(a), with
    SiLU'(a) = sig(a) (1 + a (1 - sig(a))).  Returns (h, da, du), float64."""
    a, u, dh = _f64(a), _f64(u), _f64(dh)
    sig = 1.0 / (1.0 + np.exp(-a))
    h = a * sig * u
    return h, dh * u * sig * (1.0 + a * (1.0 - sig)), dh * a * sig


def expert_ffn_backward(X, w_gate_e, w_up_e, w_down_e, dY):
    """Backward of y = (SiLU(a) * u) Wd^T with a = X Wg^T, u = X Wu^T:
    each product C = A B gives dA = dC B^T and dB = A^T dC ([V4-overlap], PP
    bubble section: a layer's backward turns dy into dx and dW = x^T dy);
    SiLU'(a) = sig(a) (1 + a (1 - sig(a))).  Returns
    (dX, dWg, dWu, dWd, dict of the intermediates a, u, h, dh, da, du)."""
    X, Wg, Wu, Wd, dY = (_f64(v) for v in (X, w_gate_e, w_up_e, w_down_e, dY))
    a = X @ Wg.T
    u = X @ Wu.T
    dh = dY @ Wd                      # y = h Wd^T
    h, da, du = swiglu_backward(a, u, dh)
    dWd = dY.T @ h
    dX = da @ Wg + du @ Wu
    dWg = da.T @ X
    dWu = du.T @ X
    return dX, dWg, dWu, dWd, dict(a=a, u=u, h=h, dh=dh, da=da, du=du)


def grouped_ffn_backward(x_perm, offsets, w_gate, w_up, w_down, dy_perm):
    """Every expert's backward on its own row segment; experts without rows
    get zero weight gradients."""
    x_perm = _f64(x_perm)
    E = len(offsets) - 1
    dx = np.zeros_like(x_perm)
    dwg = np.zeros(np.shape(w_gate))
    dwu = np.zeros(np.shape(w_up))
    dwd = np.zeros(np.shape(w_down))
    A, f = x_perm.shape[0], np.shape(w_gate)[1]
    inter = {n: np.zeros((A, f)) for n in ("a", "u", "h", "dh", "da", "du")}
    dy = _f64(dy_perm)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            dx[r0:r1], dwg[e], dwu[e], dwd[e], it = expert_ffn_backward(
                x_perm[r0:r1], w_gate[e], w_up[e], w_down[e], dy[r0:r1])
            for n in inter:
                inter[n][r0:r1] = it[n]
    return dx, dwg, dwu, dwd, inter


def scatter_rows_backward(dx_perm, src_of, k: int, T: int):
    """x_perm[p] = x[src_of[p] // k]  =>  dx[t] = sum of dx_perm[p] over the
    k rows p that copied token t."""
    dxp = _f64(dx_perm)
    dx = np.zeros((T, dxp.shape[1]))
    np.add.at(dx, np.asarray(src_of) // k, dxp)
    return dx


def gates_backward(s, sel, dg, k: int, presel: int = 0, renorm: int = 1):
    """Backward of `gates` with the selection held fixed (the cached routing).
    g_j = e_j / D with e_j = exp(s_j - m) and D the sum over the support set S
    (the k chosen; the P pre-selected; all E).  On S the normalised
    q_i = e_i / D has dq_i / ds_l = q_i (delta_il - q_l), and g_j = q_j for the
    k chosen, so ds_l = q_l (dq_l - sum_j g_j dg_j) on S (dq_l = dg_j when l is
    the j-th chosen expert, else 0) and ds_l = 0 off S.  The shift m cancels.
    Returns ds [T, E], float64."""
    s64 = np.asarray(s, dtype=np.float32).astype(np.float64)
    T, E = s64.shape
    sel = np.asarray(sel)
    dg = np.asarray(dg, dtype=np.float64)
    m = np.take_along_axis(s64, sel[:, :1], axis=1)
    if renorm:
        support = sel[:, :k]
    elif presel:
        support = sel[:, :presel]
    else:
        support = np.tile(np.arange(E), (T, 1))
    e_sup = np.exp(np.take_along_axis(s64, support, axis=1) - m)
    q = e_sup / e_sup.sum(axis=1, keepdims=True)
    dq_full = np.zeros((T, E))
    np.put_along_axis(dq_full, sel[:, :k], dg, axis=1)
    q_full = np.zeros((T, E))
    np.put_along_axis(q_full, support, q, axis=1)
    g = np.take_along_axis(q_full, sel[:, :k], axis=1)
    inner = np.sum(g * dg, axis=1, keepdims=True)
    ds = q_full * (dq_full - inner)
    return ds


def layer_backward(x, w_router, bias, w_gate, w_up, w_down, d_out, *, k, n_group=1,
                   topk_group=1, presel=0, renorm=1, ep_ranks=1, fwd=None) -> dict:
    """Gradients of the layer on the routing of its forward pass, which the
    backward reuses instead of routing again ([SyncTax] §2.4: the backward
    retraces the forward's routing, kept from the forward as the routing
    indices).  The selection is piecewise constant, so only the gate weights
    carry a gradient into the router: s = z + b gives dz = ds and
    db = sum_t ds[t]; z = x Wr^T gives dx += dz Wr and dWr = dz^T x.
    Returns dx, dWr, db, dWg, dWu, dWd and the intermediates."""
    if fwd is None:
        fwd = layer(x, w_router, bias, w_gate, w_up, w_down, k=k, n_group=n_group,
                    topk_group=topk_group, presel=presel, renorm=renorm, ep_ranks=ep_ranks)
    T = np.shape(x)[0]
    dy_perm, dg = combine_backward(d_out, fwd["y_perm"], fwd["slot_of"], fwd["topk_w"])
    dx_perm, dwg, dwu, dwd, inter = grouped_ffn_backward(fwd["x_perm"], fwd["offsets"], w_gate,
                                                         w_up, w_down, dy_perm)
    dx = scatter_rows_backward(dx_perm, fwd["src_of"], k, T)
    sel = select(fwd["s"], k, n_group, topk_group, presel)
    ds = gates_backward(fwd["s"], sel, dg, k, presel, renorm)
    dz = ds
    dx_router = dz @ _f64(w_router)
    dwr = dz.T @ _f64(x)
    db = dz.sum(axis=0)
    return dict(dx=dx + dx_router, dx_experts=dx, dx_router=dx_router, dw_router=dwr, d_bias=db,
                dw_gate=dwg, dw_up=dwu, dw_down=dwd, dy_perm=dy_perm, d_topk_w=dg, dz=dz,
                dx_perm=dx_perm, **inter)


# ----------------------------------------------------------------------------
# brute-force forms used to pin the above
# ----------------------------------------------------------------------------
def _best_subset(values, candidates, size):
    """The size-subset of `candidates` with the largest exact sum of `values`;
    among equal sums the lexicographically smallest sorted index tuple."""
    best, best_key = None, None
    for sub in itertools.combinations(sorted(candidates), size):
        tot = sum(Fraction(float(values[i])) for i in sub)
        key = (-tot, sub)
        if best_key is None or key < best_key:
            best, best_key = sub, key
    return best


def select_bruteforce(s, k: int, n_group: int = 1, topk_group: int = 1):
    """Chosen expert sets by exhaustive enumeration (tiny E only).

    With groups: first the topk_group-subset of groups with the largest sum of
    group maxima, then the k-subset of their experts with the largest score
    sum.  Returns a list of sorted index tuples.
    """
    s = np.asarray(s, dtype=np.float32)
    T, E = s.shape
    out = []
    for t in range(T):
        row = s[t]
        cand = range(E)
        if n_group > 1 and topk_group < n_group:
            gs = E // n_group
            gmax = [max(row[g * gs:(g + 1) * gs], key=float) for g in range(n_group)]
            keep = _best_subset(gmax, range(n_group), topk_group)
            cand = [g * gs + i for g in keep for i in range(gs)]
        out.append(_best_subset(row, cand, k))
    return out


def dense_bruteforce(x, w_router, bias, w_gate, w_up, w_down, *, k, n_group=1,
                     topk_group=1, presel=0, renorm=1):
    """out[t] = sum_e G[t, e] * FFN_e(x[t]) with a dense gate matrix G.

    Runs every expert on every token and forms no permutation, offsets or
    gather; only the routing decision is shared with `layer`.
    """
    T = np.asarray(x).shape[0]
    E = np.asarray(w_router).shape[0]
    z32 = router_logits(x, w_router).astype(np.float32)
    idx, w, _ = route(z32, bias, k=k, n_group=n_group, topk_group=topk_group,
                      presel=presel, renorm=renorm)
    G = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            G[t, idx[t, j]] += w[t, j]
    xf = _f64(x)
    out = np.zeros((T, np.asarray(w_down).shape[1]))
    for e in range(E):
        y_e, _ = expert_ffn(xf, w_gate[e], w_up[e], w_down[e])
        out += G[:, e : e + 1] * y_e
    return out
