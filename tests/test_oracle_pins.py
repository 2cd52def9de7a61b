"""Pins of the CPU oracle against things other than itself (CPU only).

Each pin is a plain function so that the mutation tests at the bottom can plant
a plausible mistake in the oracle and show that some pin catches it.
Sources of truth used here: hand-worked closed forms (tests/golden/), exhaustive
enumeration, library routines (scipy softmax, numpy stable sort, torch
SiLU/matmul), exact identities, and the pages' size/statistics statements.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import moe_oracle as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def _tied_scores(rng, T, E, levels=5):
    """float32 scores drawn from a few levels so that exact ties are common."""
    return rng.integers(-levels, levels + 1, size=(T, E)).astype(np.float32) * np.float32(0.25)


def _random_topk(rng, T, E, k):
    return np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)


# ----------------------------------------------------------------------------- pins
def pin_scores_single_add():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((50, 9)).astype(np.float32)
    b = rng.standard_normal(9).astype(np.float32)
    s = om.scores(z, b)
    # fp32 + fp32 is exact in fp64; one rounding to fp32 is the IEEE single add
    ref = (z.astype(np.float64) + b.astype(np.float64)[None, :]).astype(np.float32)
    assert s.dtype == np.float32
    assert np.array_equal(s.view(np.uint32), ref.view(np.uint32))
    neg0 = om.scores(np.array([[-0.0, 1.0]], np.float32), None)
    assert not np.signbit(neg0[0, 0])


def pin_selection_bruteforce():
    rng = np.random.default_rng(1)
    for E, k in [(4, 1), (4, 2), (6, 3), (8, 2), (8, 3)]:
        s = _tied_scores(rng, 64, E)
        sel = om.select(s, k)[:, :k]
        brute = om.select_bruteforce(s, k)
        for t in range(s.shape[0]):
            assert tuple(sorted(sel[t].tolist())) == brute[t], (E, k, t, s[t], sel[t])
            # best first, ties by index ascending
            vals = s[t, sel[t]]
            assert np.all(vals[:-1] >= vals[1:])
            for j in range(k - 1):
                if vals[j] == vals[j + 1]:
                    assert sel[t, j] < sel[t, j + 1]


def pin_group_bruteforce():
    rng = np.random.default_rng(2)
    s = _tied_scores(rng, 64, 16, levels=4)
    sel = om.select(s, 3, n_group=4, topk_group=2)[:, :3]
    brute = om.select_bruteforce(s, 3, n_group=4, topk_group=2)
    for t in range(64):
        assert tuple(sorted(sel[t].tolist())) == brute[t], (t, s[t])


def pin_group_all_kept_is_plain():
    rng = np.random.default_rng(3)
    s = rng.standard_normal((100, 32)).astype(np.float32)
    assert np.array_equal(om.select(s, 4, n_group=8, topk_group=8), om.select(s, 4))


def pin_hand_cases():
    g = _golden("hand_routing_cases.json")
    for case in g["cases"]:
        if "s" in case:
            s = np.array([case["s"]], np.float32)
            bias = None
        else:
            s = np.log(np.array([case["p"]], np.float64)).astype(np.float32)
            bias = None if case["bias_p"] is None else np.log(np.array(case["bias_p"], np.float64)).astype(np.float32)
        idx, w, _ = om.route(s, bias, k=case["k"], n_group=case["n_group"],
                             topk_group=case["topk_group"], presel=case["presel"],
                             renorm=case["renorm"])
        assert idx[0].tolist() == case["topk_idx"], case["name"]
        if "gates" in case:
            want = np.array([a / b for a, b in case["gates"]])
            assert np.max(np.abs(w[0] - want)) < 1e-6, (case["name"], w[0], want)


def pin_presel_all_is_full_softmax():
    rng = np.random.default_rng(4)
    z = rng.standard_normal((40, 12)).astype(np.float32)
    idx, w, s = om.route(z, None, k=3, presel=12, renorm=0)
    p = scipy.special.softmax(s.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(p, idx.astype(np.int64), axis=1), rtol=0, atol=1e-14)


def pin_renorm_is_softmax_then_renorm():
    rng = np.random.default_rng(5)
    for k in (1, 2, 4, 8):
        z = (2 * rng.standard_normal((30, 16))).astype(np.float32)
        idx, w, s = om.route(z, None, k=k, renorm=1)
        p = scipy.special.softmax(s.astype(np.float64), axis=1)
        pk = np.take_along_axis(p, idx.astype(np.int64), axis=1)
        assert np.allclose(w, pk / pk.sum(1, keepdims=True), rtol=1e-13, atol=0)
        assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)


def pin_gate_closed_forms():
    rng = np.random.default_rng(6)
    z = rng.standard_normal((64, 8)).astype(np.float32)
    idx, w, s = om.route(z, None, k=2, renorm=1)
    s0 = np.take_along_axis(s, idx[:, :1].astype(np.int64), 1)[:, 0].astype(np.float64)
    s1 = np.take_along_axis(s, idx[:, 1:2].astype(np.int64), 1)[:, 0].astype(np.float64)
    logistic = 1.0 / (1.0 + np.exp(s1 - s0))
    assert np.allclose(w[:, 0], logistic, rtol=1e-14, atol=0)
    assert np.allclose(w[:, 1], 1.0 - logistic, rtol=0, atol=1e-14)
    idx1, w1, _ = om.route(z, None, k=1, renorm=1)
    assert np.array_equal(w1, np.ones_like(w1))
    assert np.array_equal(idx1[:, 0], np.argmax(z, axis=1))


def pin_permute_invariants():
    rng = np.random.default_rng(7)
    T, E, k, R = 1000, 16, 4, 4
    idx = _random_topk(rng, T, E, k)
    p = om.permute(idx, E, R)
    A = T * k
    assert p["counts"].sum() == A
    assert p["offsets"][0] == 0 and p["offsets"][-1] == A
    assert np.array_equal(np.diff(p["offsets"]), p["counts"])
    assert sorted(p["slot_of"].tolist()) == list(range(A))          # bijection
    assert np.array_equal(p["src_of"][p["slot_of"]], np.arange(A))  # slot_of o src_of = id
    assert np.array_equal(p["slot_of"][p["src_of"]], np.arange(A))
    flat = idx.reshape(-1)
    for e in range(E):
        seg = p["src_of"][p["offsets"][e]:p["offsets"][e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg // k) > 0)  # ascending token order within an expert
    assert np.array_equal(p["rank_offsets"], p["offsets"][[0, 4, 8, 12, 16]])


def pin_permute_is_stable_sort():
    rng = np.random.default_rng(8)
    for T, E, k in [(7, 3, 2), (300, 8, 2), (257, 64, 8)]:
        idx = _random_topk(rng, T, E, k)
        p = om.permute(idx, E)
        # a stable sort of the flattened expert ids lists the entries in slot order
        assert np.array_equal(p["src_of"], np.argsort(idx.reshape(-1), kind="stable"))


def pin_call_count():
    g = _golden("routing_call_count.json")
    rng = np.random.default_rng(9)
    idx = _random_topk(rng, g["T"], g["E"], g["k"])
    p = om.permute(idx, g["E"], g["ep_ranks"])
    assert int(p["counts"].sum()) == g["expected_expert_calls"]
    assert idx.astype(np.int32).nbytes == g["expected_index_bytes"]
    assert len(p["rank_offsets"]) == g["ep_ranks"] + 1
    assert p["rank_offsets"][1] == p["offsets"][g["E"] // g["ep_ranks"]]


def pin_swiglu_unit():
    g = _golden("swiglu_unit_case.json")
    y, h = om.expert_ffn(np.array(g["x"]), np.array(g["w_gate"])[0], np.array(g["w_up"])[0],
                         np.array(g["w_down"])[0])
    assert np.allclose(h, g["h"], rtol=1e-15, atol=0)
    assert np.allclose(y, g["y"], rtol=1e-15, atol=0)


def _torch_mlp(x, wg, wu, wd):
    x, wg, wu, wd = (torch.from_numpy(np.asarray(a, np.float64)) for a in (x, wg, wu, wd))
    return (torch.nn.functional.silu(x @ wg.T) * (x @ wu.T) @ wd.T).numpy()


def pin_single_expert_is_dense_mlp():
    rng = np.random.default_rng(10)
    T, d, f = 33, 24, 40
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((1, d))
    wg, wu, wd = (0.2 * rng.standard_normal(s) for s in ((1, f, d), (1, f, d), (1, d, f)))
    r = om.layer(x, wr, None, wg, wu, wd, k=1)
    assert np.allclose(r["out"], _torch_mlp(x, wg[0], wu[0], wd[0]), rtol=1e-12, atol=1e-12)


def pin_identical_experts():
    rng = np.random.default_rng(11)
    T, d, f, E, k = 50, 16, 24, 6, 3
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d))
    one = [0.3 * rng.standard_normal(s) for s in ((f, d), (f, d), (d, f))]
    wg, wu, wd = (np.repeat(a[None], E, axis=0) for a in one)
    r = om.layer(x, wr, None, wg, wu, wd, k=k, renorm=1)
    assert np.allclose(r["out"], _torch_mlp(x, *one), rtol=1e-12, atol=1e-12)


def pin_combine_identity_experts():
    rng = np.random.default_rng(12)
    T, d, E = 80, 8, 8
    x = rng.standard_normal((T, d))
    for k in (1, 2, 3):
        z = rng.standard_normal((T, E)).astype(np.float32)
        idx, w, _ = om.route(z, None, k=k, renorm=1)
        p = om.permute(idx, E)
        out = om.combine(om.gather_rows(x, p["src_of"], k), p["slot_of"], w)
        if k == 1:
            assert np.array_equal(out, x)
        else:
            assert np.allclose(out, x, rtol=1e-14, atol=1e-14)


ROUTING_MODES = [
    dict(E=8, k=2),
    dict(E=8, k=2, bias="normal"),
    dict(E=12, k=2, presel=8, renorm=0),
    dict(E=16, k=3, n_group=4, topk_group=2),
    dict(E=6, k=2, renorm=0),
]


def _small_problem(rng, E, T=24, d=12, f=20, bias=None):
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d))
    b = rng.standard_normal(E).astype(np.float32) if bias == "normal" else None
    wg, wu, wd = (0.3 * rng.standard_normal(s) for s in ((E, f, d), (E, f, d), (E, d, f)))
    return x, wr, b, wg, wu, wd


def _mode_kw(m):
    return {k: v for k, v in m.items() if k in ("k", "n_group", "topk_group", "presel", "renorm")}


def pin_layer_matches_dense_bruteforce():
    rng = np.random.default_rng(13)
    for m in ROUTING_MODES:
        prob = _small_problem(rng, m["E"], bias=m.get("bias"))
        r = om.layer(*prob, **_mode_kw(m))
        dense = om.dense_bruteforce(*prob, **_mode_kw(m))
        assert np.allclose(r["out"], dense, rtol=1e-12, atol=1e-12), m


def pin_token_permutation():
    rng = np.random.default_rng(14)
    for m in ROUTING_MODES:
        x, wr, b, wg, wu, wd = _small_problem(rng, m["E"], bias=m.get("bias"))
        perm = rng.permutation(x.shape[0])
        r1 = om.layer(x, wr, b, wg, wu, wd, **_mode_kw(m))
        r2 = om.layer(x[perm], wr, b, wg, wu, wd, **_mode_kw(m))
        assert np.allclose(r2["out"], r1["out"][perm], rtol=1e-12, atol=1e-12), m


def pin_expert_relabel():
    rng = np.random.default_rng(15)
    for m in ROUTING_MODES:
        E = m["E"]
        x, wr, b, wg, wu, wd = _small_problem(rng, E, bias=m.get("bias"))
        ng = m.get("n_group", 1)
        gs = E // ng
        # permute whole groups, and experts inside each group
        gperm = rng.permutation(ng)
        relabel = np.concatenate([g * gs + rng.permutation(gs) for g in gperm])
        bb = None if b is None else b[relabel]
        r1 = om.layer(x, wr, b, wg, wu, wd, **_mode_kw(m))
        r2 = om.layer(x, wr[relabel], bb, wg[relabel], wu[relabel], wd[relabel], **_mode_kw(m))
        assert np.allclose(r2["out"], r1["out"], rtol=1e-12, atol=1e-12), m
        assert np.array_equal(np.sort(relabel[r2["topk_idx"]], 1), np.sort(r1["topk_idx"], 1))


def pin_margins():
    s = np.array([[3.0, 1.0, 2.0, 1.5]])
    assert om.margins(s, 2)[0] == pytest.approx(0.5)
    g = np.array([[5.0, 0.0, 4.9, 4.8, 0.0, 0.0, 4.85, 4.0]])
    # experts in kept groups: 5, 0, 4.9, 4.8 -> 3rd/4th gap 4.8 - 0 = 4.8; group gap 4.9 - 4.85
    assert om.margins(g, 3, n_group=4, topk_group=2)[0] == pytest.approx(0.05)


def pin_routing_statistics():
    g = _golden("routing_statistics.json")
    rng = np.random.default_rng(16)
    z = rng.standard_normal((40000, 64)).astype(np.float32)
    idx, _, _ = om.route(z, None, k=2)
    share = np.bincount(idx.ravel(), minlength=64) / idx.size
    assert abs(share.mean() - g["uniform_share_E64"]) < 1e-12
    assert np.max(np.abs(share - g["uniform_share_E64"])) < 0.0025
    z = rng.standard_normal((40000, 16)).astype(np.float32)
    idx, _, _ = om.route(z, None, k=2)
    p = np.bincount(idx.ravel(), minlength=16) / idx.size
    ent = -(p * np.log2(p)).sum()
    assert g["max_entropy_bits_E16"] - 0.01 < ent <= g["max_entropy_bits_E16"] + 1e-12


def pin_route_stats_closed_forms():
    g = _golden("routing_statistics.json")
    # equal scores: softmax is 1/E, entropy log2 E, the top-P keep P/E of the mass
    z = np.zeros((5, 16), np.float32)
    idx = np.tile(np.arange(16, dtype=np.int32).reshape(8, 2), (1, 1))[:5]
    r = om.route_stats(z, None, idx, 16, presel=4)
    assert r["token_entropy_bits"] == pytest.approx(g["max_entropy_bits_E16"], abs=1e-12)
    assert r["presel_gap"] == pytest.approx(0.75, abs=1e-12)
    # one dominant expert: entropy and gap vanish
    z = np.zeros((3, 8), np.float32)
    z[:, 3] = 60.0
    r = om.route_stats(z, None, np.array([[3, 0]] * 3, np.int32), 8, presel=1)
    assert r["token_entropy_bits"] < 1e-20 and r["presel_gap"] < 1e-20
    # the bias enters the scores: a bias that cancels z gives equal scores
    zb = np.array([[1.0, -1.0, 0.5, 0.0]], np.float32)
    r = om.route_stats(zb, -zb[0], np.array([[0, 1]], np.int32), 4, presel=2)
    assert r["token_entropy_bits"] == pytest.approx(2.0, abs=1e-12)
    assert r["presel_gap"] == pytest.approx(0.5, abs=1e-12)
    # an even histogram: load entropy log2 E (the pages' ideal: 4.0 bits for
    # 16 experts), every share 1/E, maximum load ratio 1
    idx = np.arange(64, dtype=np.int32).reshape(32, 2) % 16
    r = om.route_stats(np.zeros((32, 16), np.float32), None, idx, 16, ep_ranks=4)
    assert r["load_entropy_bits"] == pytest.approx(g["max_entropy_bits_E16"], abs=1e-12)
    assert r["max_load_ratio"] == pytest.approx(1.0)
    assert r["hist"].tolist() == [4] * 16 and r["rank_load"].tolist() == [16] * 4
    # every token on the same k = 2 experts: log2 k bits, ratio E / k
    idx = np.tile(np.array([[5, 9]], np.int32), (7, 1))
    r = om.route_stats(np.zeros((7, 12), np.float32), None, idx, 12, ep_ranks=3)
    assert r["load_entropy_bits"] == pytest.approx(1.0, abs=1e-12)
    assert r["max_load_ratio"] == pytest.approx(6.0)
    assert r["hist"][5] == 7 and r["hist"][9] == 7 and r["hist"].sum() == 14
    assert r["rank_load"].tolist() == [0, 7, 7]
    # no tokens: zeros
    r = om.route_stats(np.zeros((0, 4), np.float32), None, np.zeros((0, 2), np.int32), 4)
    assert r["load_entropy_bits"] == 0.0 and r["token_entropy_bits"] == 0.0


def pin_fp8_e4m3_codes():
    """The E4M3 format's own fixed points and rounding ([SyncTax] §3.1 FP8)."""
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = om.fp8_e4m3_decode(finite)
    # every finite code encodes its own value back (-0 keeps its sign bit)
    assert np.array_equal(om.fp8_e4m3_encode(vals.astype(np.float32)), finite)
    # the magnitudes are strictly increasing with the code
    pos = vals[finite < 0x80]
    assert np.all(np.diff(pos) > 0)
    fixed = {448.0: 0x7E, -448.0: 0xFE, 1.0: 0x38, 2.0 ** -9: 0x01, 2.0 ** -6: 0x08,
             0.9375: 0x37, 240.0: 0x77, 0.0: 0x00}
    for v, c in fixed.items():
        assert int(om.fp8_e4m3_encode(np.float32(v))) == c, (v, c)
    # ties go to the even code: 1 + 1/16 -> 1.0, 1 + 3/16 -> 1.25, 2^-10 -> 0, 3 2^-10 -> 2^-8
    ties = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02}
    for v, c in ties.items():
        assert int(om.fp8_e4m3_encode(np.float32(v))) == c, (v, c)


def pin_fp8_row_quantization():
    bits = om.round_bf16(np.array([[-3.0, 5.0, 1.0, 2.0], [0.75] * 4], np.float32))
    codes, s, z = om.quantize_rows_fp8(bits)
    # row 0: centre 1, half-range 4: the extremes land on -+448, the centre on 0
    assert z[0] == 1.0 and s[0] == np.float32(4.0) / np.float32(448.0)
    assert codes[0, 0] == 0xFE and codes[0, 1] == 0x7E and codes[0, 2] == 0x00
    # 2.0 maps to 112 = 1.75 * 2^6 (E4M3 exact)
    assert codes[0, 3] == 0x6E
    # a constant row: scale 0, codes 0, and it comes back exactly
    assert s[1] == 0.0 and not codes[1].any()
    back = om.dequantize_rows_fp8(codes, s, z)
    assert np.array_equal(back[1], bits[1])
    # bf16 rounding of the decode: even ties
    assert om.round_bf16(np.float32(1.0 + 2.0 ** -8)).item() == 0x3F80
    assert om.round_bf16(np.float32(1.0 + 3 * 2.0 ** -8)).item() == 0x3F82
    # error bound on random rows: E4M3 keeps 3 mantissa bits of v, so
    # |x - x^| <= half-range / 16 (plus the bf16 rounding of x^)
    rng = np.random.default_rng(5)
    x = om.round_bf16(rng.standard_normal((64, 96)).astype(np.float32))
    codes, s, z = om.quantize_rows_fp8(x)
    xf = om.widen_bf16(x)
    xr = om.widen_bf16(om.dequantize_rows_fp8(codes, s, z))
    hr = s.astype(np.float64) * 448.0
    assert np.all(np.abs(xr - xf) <= hr[:, None] / 16 + np.abs(xf) * 2.0 ** -8 + 1e-30)


def pin_fp8_weight_quantization():
    """Per-output-channel E4M3 weights: each row's largest magnitude lands on
    +-448 exactly (codes 0x7E / 0xFE), power-of-two ratios to it stay exact,
    an all-zero row has scale 0 and zero codes, and the decoded weight is
    within half an E4M3 step of the weight (3 mantissa bits: 2^-4 |v| for
    normal codes, 2^-10 below 2^-6)."""
    w = np.array([[1.0, -2.0, 0.5, 2.0, 0.25],
                  [0.0, 0.0, 0.0, 0.0, 0.0],
                  [-3.0, 0.75, 1.5, -0.375, 3.0]], np.float32)
    codes, s = om.quantize_weights_fp8(w)
    assert s.dtype == np.float32 and codes.dtype == np.uint8
    assert s[0] == np.float32(2.0) / np.float32(448.0) and s[1] == 0.0
    assert s[2] == np.float32(3.0) / np.float32(448.0)
    # row 0: -2 and 2 are the extremes; 1 = 224, 0.5 = 112, 0.25 = 56 are exact E4M3 values
    assert codes[0].tolist() == [0x76, 0xFE, 0x6E, 0x7E, 0x66]
    assert not codes[1].any()
    # row 2: 3 -> 448, -3 -> -448, 1.5 -> 224, 0.75 -> 112, -0.375 -> -56
    assert codes[2].tolist() == [0xFE, 0x6E, 0x76, 0xE6, 0x7E]
    rng = np.random.default_rng(43)
    bits = om.round_bf16((0.02 * rng.standard_normal((3, 24, 200))).astype(np.float32))
    codes, s = om.quantize_weights_fp8(bits)
    assert codes.shape == bits.shape and s.shape == (3, 24)
    wv = om.widen_bf16(bits)
    back = om.fp8_e4m3_decode(codes) * s.astype(np.float64)[..., None]
    v = np.abs(wv) / s.astype(np.float64)[..., None]
    step = np.where(v >= 2.0 ** -6, 2.0 ** -4 * v, 2.0 ** -10) * s.astype(np.float64)[..., None]
    assert np.all(np.abs(back - wv) <= step * (1 + 1e-6))
    # the row maximum is +-448 in every row
    assert np.all(np.max(np.abs(om.fp8_e4m3_decode(codes)), axis=-1) == 448.0)


def pin_gate_up_fp8_on_exact_operands():
    """When the FP8 operands decode to values that the bf16 path can hold
    exactly, the FP8 first GEMM is the pinned SwiGLU first GEMM (expert_ffn)
    on those values; a shift of every token row by c moves a by
    c * sum_k w^[n, k] (the zero point enters linearly)."""
    rng = np.random.default_rng(44)
    T, F, K = 9, 6, 40
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F and ((c >> 3) & 0xF) <= 9],
                      np.uint8)
    xc = rng.choice(finite, size=(T, K))
    gc, uc = rng.choice(finite, size=(F, K)), rng.choice(finite, size=(F, K))
    xs = np.full(T, 0.5, np.float32)            # powers of two: x^ = code s + z stays exact
    xz = np.array([0.0, 0.25, -1.0, 2.0, 0.0, -0.5, 1.0, 0.125, 0.0], np.float32)
    gs, us = np.full(F, 0.25, np.float32), np.full(F, 2.0 ** -5, np.float32)
    h, a, u = om.gate_up_fp8(xc, xs, xz, gc, gs, uc, us)
    xd = om.fp8_e4m3_decode(xc) * 0.5 + xz.astype(np.float64)[:, None]
    wg = om.fp8_e4m3_decode(gc) * 0.25
    wu = om.fp8_e4m3_decode(uc) * 2.0 ** -5
    _, h_ref = om.expert_ffn(xd, wg, wu, np.zeros((3, F)))
    assert np.allclose(h, h_ref, rtol=1e-13, atol=1e-13)
    assert np.allclose(a, xd @ wg.T, rtol=1e-13, atol=1e-13)
    # zero point: shifting every row by c adds c * sum_k w^[n, k] to a
    h2, a2, _ = om.gate_up_fp8(xc, xs, xz + np.float32(0.75), gc, gs, uc, us)
    assert np.allclose(a2 - a, 0.75 * wg.sum(axis=1)[None, :], rtol=1e-12, atol=1e-12)


def pin_router_logits_hand_case():
    """z = x Wr^T on a hand-worked case whose last logit needs 33 significant
    bits (exact in float64, rounded by any float32 accumulation), given both
    as float64 values and as the bf16 bit patterns of the same values."""
    g = _golden("router_logits_case.json")
    want = np.array(g["z"], dtype=np.float64)
    z = om.router_logits(np.array(g["x"]), np.array(g["w_router"]))
    assert z.shape == want.shape and np.array_equal(z, want), z
    zb = om.router_logits(np.array(g["x_bf16_bits"], np.uint16),
                          np.array(g["w_router_bf16_bits"], np.uint16))
    assert np.array_equal(zb, want), zb


def _bf16_values_torch(bits):
    """bf16 bit patterns -> float64 through torch's own bfloat16 type (not the
    oracle's widening)."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(bits, np.uint16)).view(np.int16).copy())
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def _random_bf16_bits(rng, shape, spread=12):
    """bf16 bit patterns of values with random signs, exponents over `spread`
    binades and all 7 mantissa bits set at random."""
    sign = rng.integers(0, 2, size=shape, dtype=np.uint16) << 15
    expo = (127 - spread // 2 + rng.integers(0, spread, size=shape)).astype(np.uint16) << 7
    mant = rng.integers(0, 128, size=shape, dtype=np.uint16)
    return (sign | expo | mant).astype(np.uint16)


def pin_router_logits_exact_sum():
    """Every logit against its exact rational value (brute-force triple loop
    in Fractions), within the float64 summation bound d u sum|x w|."""
    rng = np.random.default_rng(40)
    T, E, d = 6, 5, 9
    xb, wb = _random_bf16_bits(rng, (T, d)), _random_bf16_bits(rng, (E, d))
    xv, wv = _bf16_values_torch(xb), _bf16_values_torch(wb)
    z = om.router_logits(xb, wb)
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(float(xv[t, i])) * Fraction(float(wv[e, i])) for i in range(d))
            bound = d * 2.0 ** -53 * float(np.sum(np.abs(xv[t] * wv[e])))
            assert abs(Fraction(float(z[t, e])) - exact) <= Fraction(bound), (t, e)


def pin_bf16_bit_patterns_are_their_values():
    """Every bf16 workload feeds the oracle uint16 bit patterns.  Routing,
    FFN, combine and the whole layer must give exactly what they give on the
    same numbers widened by torch's bfloat16 type and passed as float64."""
    rng = np.random.default_rng(41)
    T, d, f = 40, 16, 24
    for m in ROUTING_MODES:
        E = m["E"]
        bits = dict(x=_random_bf16_bits(rng, (T, d), 6),
                    w_router=_random_bf16_bits(rng, (E, d), 6),
                    w_gate=_random_bf16_bits(rng, (E, f, d), 6),
                    w_up=_random_bf16_bits(rng, (E, f, d), 6),
                    w_down=_random_bf16_bits(rng, (E, d, f), 6))
        vals = {n: _bf16_values_torch(b) for n, b in bits.items()}
        b = rng.standard_normal(E).astype(np.float32) if m.get("bias") else None
        rb = om.layer(bits["x"], bits["w_router"], b, bits["w_gate"], bits["w_up"],
                      bits["w_down"], **_mode_kw(m))
        rv = om.layer(vals["x"], vals["w_router"], b, vals["w_gate"], vals["w_up"],
                      vals["w_down"], **_mode_kw(m))
        for n in ("logits", "topk_idx", "topk_w", "h", "y_perm", "out"):
            assert np.array_equal(rb[n], rv[n]), (m, n)
        assert np.array_equal(_bf16_values_torch(rb["x_perm"]), rv["x_perm"]), m
        # the combine alone on bf16 expert outputs
        yb = _random_bf16_bits(rng, (T * m["k"], d), 6)
        cb = om.combine(yb, rb["slot_of"], rb["topk_w"])
        cv = om.combine(_bf16_values_torch(yb), rb["slot_of"], rb["topk_w"])
        assert np.array_equal(cb, cv), m


def pin_widen_bf16():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4049, 0x7F7F], np.uint16)
    got = om.widen_bf16(bits)
    want = [1.0, -1.0, 0.0, -0.0, 3.140625, float.fromhex("0x1.fep127")]
    assert got.tolist() == want


def _fd_problem(rng, m):
    T, d, f = 10, 6, 5
    x, wr, b, wg, wu, wd = _small_problem(rng, m["E"], T=T, d=d, f=f, bias=m.get("bias"))
    return [x, wr, b, wg, wu, wd], rng.standard_normal((T, d))


def pin_layer_backward_finite_differences():
    """Each gradient of layer_backward against a central difference of the
    (separately pinned) forward along a random direction, in every routing
    mode; the routing must not change inside the step."""
    rng = np.random.default_rng(41)
    eps = 1e-3
    names = ["dx", "dw_router", "d_bias", "dw_gate", "dw_up", "dw_down"]
    for m in ROUTING_MODES:
        params, R = _fd_problem(rng, m)
        kw = _mode_kw(m)
        g = om.layer_backward(*params, R, **kw)
        base = om.layer(*params, **kw)["topk_idx"]
        for i, name in enumerate(names):
            if params[i] is None:
                continue
            v = rng.standard_normal(np.shape(params[i]))
            f_at = []
            for sgn in (1.0, -1.0):
                pp = list(params)
                pp[i] = np.asarray(params[i], np.float64) + sgn * eps * v
                r = om.layer(*pp, **kw)
                assert np.array_equal(r["topk_idx"], base), (m, name)
                f_at.append(np.sum(r["out"] * R))
            fd = (f_at[0] - f_at[1]) / (2 * eps)
            an = float(np.sum(g[name] * v))
            assert abs(fd - an) <= 2e-4 * max(1.0, abs(fd)), (m, name, fd, an)


def pin_expert_backward_matches_autograd():
    """One expert's backward against torch autograd of the same MLP (float64)."""
    rng = np.random.default_rng(42)
    X = rng.standard_normal((7, 9))
    wg, wu, wd = rng.standard_normal((5, 9)), rng.standard_normal((5, 9)), rng.standard_normal((9, 5))
    dY = rng.standard_normal((7, 9))
    dX, dWg, dWu, dWd, _ = om.expert_ffn_backward(X, wg, wu, wd, dY)
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (X, wg, wu, wd)]
    y = torch.nn.functional.silu(t[0] @ t[1].T) * (t[0] @ t[2].T) @ t[3].T
    y.backward(torch.tensor(dY))
    for mine, ref in zip((dX, dWg, dWu, dWd), t):
        assert np.allclose(mine, ref.grad.numpy(), rtol=1e-12, atol=1e-12)


def pin_gates_backward_matches_autograd():
    """Softmax-gate backward against torch autograd of a softmax over the
    support set, gathered at the chosen experts, in each gate mode."""
    rng = np.random.default_rng(43)
    T, E, k = 6, 10, 3
    s = rng.standard_normal((T, E)).astype(np.float32)
    dg = rng.standard_normal((T, k))
    for presel, renorm in ((0, 1), (6, 0), (0, 0), (6, 1)):
        sel = om.select(s, k, presel=presel)
        ds = om.gates_backward(s, sel, dg, k, presel, renorm)
        st = torch.tensor(s.astype(np.float64), requires_grad=True)
        supp = sel[:, :k] if renorm else (sel[:, :presel] if presel else np.tile(np.arange(E), (T, 1)))
        sup_t = torch.tensor(supp, dtype=torch.long)
        q = torch.softmax(torch.gather(st, 1, sup_t), dim=1)
        qf = torch.zeros(T, E, dtype=torch.float64).scatter(1, sup_t, q)
        g = torch.gather(qf, 1, torch.tensor(sel[:, :k], dtype=torch.long))
        g.backward(torch.tensor(dg))
        assert np.allclose(ds, st.grad.numpy(), rtol=1e-12, atol=1e-14), (presel, renorm)
        assert np.allclose(ds.sum(axis=1), 0.0, atol=1e-12)  # softmax shift invariance


def pin_gates_backward_two_choice_closed_form():
    """Top-2 with renormalisation: g1 = sigmoid(s1 - s2), g2 = 1 - g1, so
    ds1 = g1 g2 (dg1 - dg2) = -ds2 and every other expert gets nothing."""
    rng = np.random.default_rng(45)
    T, E = 9, 7
    s = rng.standard_normal((T, E)).astype(np.float32)
    dg = rng.standard_normal((T, 2))
    sel = om.select(s, 2)
    ds = om.gates_backward(s, sel, dg, 2, 0, 1)
    s64 = s.astype(np.float64)
    for t in range(T):
        e1, e2 = int(sel[t, 0]), int(sel[t, 1])
        g1 = 1.0 / (1.0 + math.exp(-(s64[t, e1] - s64[t, e2])))
        want = g1 * (1.0 - g1) * (dg[t, 0] - dg[t, 1])
        assert math.isclose(ds[t, e1], want, rel_tol=1e-12, abs_tol=1e-15)
        assert math.isclose(ds[t, e2], -want, rel_tol=1e-12, abs_tol=1e-15)
        others = [e for e in range(E) if e not in (e1, e2)]
        assert np.all(ds[t, others] == 0)


def pin_single_choice_router_has_no_gradient():
    """k = 1 with renormalisation: the gate is 1 whatever the scores, so the
    router gets no gradient at all."""
    rng = np.random.default_rng(44)
    x, wr, b, wg, wu, wd = _small_problem(rng, 5, T=8, d=6, f=4)
    g = om.layer_backward(x, wr, b, wg, wu, wd, rng.standard_normal((8, 6)), k=1)
    assert np.all(g["dz"] == 0) and np.all(g["dw_router"] == 0) and np.all(g["dx_router"] == 0)


PINS = {name: fn for name, fn in globals().items() if name.startswith("pin_")}


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    PINS[name]()


# ------------------------------------------------------------------ planted mistakes
def _ties_to_highest(v):
    n = v.shape[-1]
    return (n - 1) - np.argsort(-v[..., ::-1], axis=-1, kind="stable")


def _scores_without_bias(z32, bias=None):
    return np.asarray(z32, dtype=np.float32) + np.float32(0.0)


def _gates_presel_uses_k(s, sel, k, presel=0, renorm=1):
    return _ORIG["gates"](s, sel, k, 0, 1)


def _silu_wrong_branch(X, wg, wu, wd):
    X = om._f64(X)
    h = (X @ om._f64(wg).T) * om.silu(X @ om._f64(wu).T)
    return h @ om._f64(wd).T, h


def _permute_reversed_within_expert(topk_idx, E, ep_ranks=1):
    p = _ORIG["permute"](topk_idx, E, ep_ranks)
    src = p["src_of"].copy()
    for e in range(E):
        a, b = p["offsets"][e], p["offsets"][e + 1]
        src[a:b] = src[a:b][::-1]
    slot = np.empty_like(src)
    slot[src] = np.arange(src.size)
    p.update(src_of=src, slot_of=slot)
    return p


def _combine_swapped_gates(y_perm, slot_of, topk_w):
    return _ORIG["combine"](y_perm, slot_of, np.asarray(topk_w)[:, ::-1])


def _eligible_mean_group(s, n_group, topk_group):
    T, E = s.shape
    if n_group <= 1 or topk_group >= n_group:
        return np.ones((T, E), dtype=bool)
    gs = E // n_group
    kept = om._order_desc(s.reshape(T, n_group, gs).mean(axis=2))[:, :topk_group]
    gmask = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(gmask, kept, True, axis=1)
    return np.repeat(gmask, gs, axis=1)


def _rank_offsets_by_rank_index(topk_idx, E, ep_ranks=1):
    p = _ORIG["permute"](topk_idx, E, ep_ranks)
    p["rank_offsets"] = p["offsets"][: ep_ranks + 1].copy()
    return p


def _gates_no_max_exp_sign(s, sel, k, presel=0, renorm=1):
    w = _ORIG["gates"](s, sel, k, presel, renorm)
    return w[:, ::-1].copy()


_ORIG = {n: getattr(om, n) for n in ("gates", "permute", "combine")}

def _route_stats_natural_log(logits32, bias, topk_idx, E, ep_ranks=1, presel=0):
    r = _ORIG_ROUTE_STATS(logits32, bias, topk_idx, E, ep_ranks, presel)
    r["load_entropy_bits"] *= np.log(2.0)
    r["token_entropy_bits"] *= np.log(2.0)
    return r


def _route_stats_first_choice_only(logits32, bias, topk_idx, E, ep_ranks=1, presel=0):
    return _ORIG_ROUTE_STATS(logits32, bias, np.asarray(topk_idx)[:, :1], E, ep_ranks, presel)


_ORIG_ROUTE_STATS = om.route_stats


def _fp8_round_half_up(v):
    v = np.asarray(v, np.float32)
    orig = np.rint
    try:
        np_rint = lambda y: np.floor(np.asarray(y) + np.float32(0.5))
        om.np.rint = np_rint
        return _ORIG_FP8_ENCODE(v)
    finally:
        om.np.rint = orig


def _quantize_full_range_scale(x_bits):
    x = om.widen_bf16(np.asarray(x_bits, dtype=np.uint16)).astype(np.float32)
    hi, lo = x.max(1), x.min(1)
    z = ((hi + lo) * np.float32(0.5)).astype(np.float32)
    s = ((hi - lo) / np.float32(448.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(s[:, None] > 0, (x - z[:, None]) / s[:, None], np.float32(0.0)).astype(np.float32)
    return om.fp8_e4m3_encode(np.clip(v, -448, 448)), s, z


def _expert_bwd_silu_prime_dropped(X, w_gate_e, w_up_e, w_down_e, dY):
    X, Wg, Wu, Wd, dY = (np.asarray(v, np.float64) for v in (X, w_gate_e, w_up_e, w_down_e, dY))
    a, u = X @ Wg.T, X @ Wu.T
    sig = 1.0 / (1.0 + np.exp(-a))
    h = a * sig * u
    dh = dY @ Wd
    da, du = dh * u * sig, dh * a * sig
    return (da @ Wg + du @ Wu, da.T @ X, du.T @ X, dY.T @ h,
            dict(a=a, u=u, h=h, dh=dh, da=da, du=du))


def _expert_bwd_branches_swapped(X, w_gate_e, w_up_e, w_down_e, dY):
    dX, dWg, dWu, dWd, it = _ORIG_EXPERT_BWD(X, w_gate_e, w_up_e, w_down_e, dY)
    return dX, dWu, dWg, dWd, it


def _gates_bwd_sign(s, sel, dg, k, presel=0, renorm=1):
    return -_ORIG_GATES_BWD(s, sel, dg, k, presel, renorm)


def _combine_bwd_no_gate(d_out, y_perm, slot_of, topk_w):
    dy, dg = _ORIG_COMBINE_BWD(d_out, y_perm, slot_of, np.ones_like(np.asarray(topk_w)))
    return dy, _ORIG_COMBINE_BWD(d_out, y_perm, slot_of, topk_w)[1]


def _scatter_bwd_first_row_only(dx_perm, src_of, k, T):
    dxp = np.asarray(dx_perm, np.float64)
    dx = np.zeros((T, dxp.shape[1]))
    src = np.asarray(src_of)
    keep = src % k == 0
    np.add.at(dx, src[keep] // k, dxp[keep])
    return dx


def _router_logits_fp32_accumulate(x, w_router):
    return (om._f64(x).astype(np.float32) @ om._f64(w_router).astype(np.float32).T).astype(np.float64)


def _router_logits_scaled(x, w_router):
    xf = om._f64(x)
    return (xf @ om._f64(w_router).T) / math.sqrt(xf.shape[1])


def _f64_without_widening(a):
    return np.asarray(a).astype(np.float64)


def _swiglu_bwd_du_without_sigmoid(a, u, dh):
    h, da, _ = _ORIG_SWIGLU_BWD(a, u, dh)
    return h, da, om._f64(dh) * om._f64(a)


def _fp8_weight_scale_per_column(w):
    a = np.asarray(w)
    x = (om.widen_bf16(a) if a.dtype == np.uint16 else a.astype(np.float64)).astype(np.float32)
    s = (np.abs(x).max(axis=-2) / np.float32(om.F8_MAX)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(s[..., None, :] > 0, x / s[..., None, :], np.float32(0.0)).astype(np.float32)
    return om.fp8_e4m3_encode(np.clip(v, -448, 448).astype(np.float32)), s


def _gate_up_fp8_no_zero_point(x_codes, x_scale, x_zero, wg_codes, wg_scale, wu_codes, wu_scale):
    return _ORIG_GATE_UP_FP8(x_codes, x_scale, np.zeros_like(np.asarray(x_zero)), wg_codes,
                             wg_scale, wu_codes, wu_scale)


_ORIG_EXPERT_BWD = om.expert_ffn_backward
_ORIG_SWIGLU_BWD = om.swiglu_backward
_ORIG_GATE_UP_FP8 = om.gate_up_fp8
_ORIG_GATES_BWD = om.gates_backward
_ORIG_COMBINE_BWD = om.combine_backward
_ORIG_FP8_ENCODE = om.fp8_e4m3_encode

MUTANTS = {
    "ties-to-highest-index": ("_order_desc", _ties_to_highest),
    "bias-dropped": ("scores", _scores_without_bias),
    "presel-denominator-over-k": ("gates", _gates_presel_uses_k),
    "silu-on-up-branch": ("expert_ffn", _silu_wrong_branch),
    "permute-not-stable": ("permute", _permute_reversed_within_expert),
    "combine-gates-swapped": ("combine", _combine_swapped_gates),
    "group-score-mean": ("_eligible", _eligible_mean_group),
    "rank-offsets-wrong": ("permute", _rank_offsets_by_rank_index),
    "gates-reversed": ("gates", _gates_no_max_exp_sign),
    "stats-entropy-in-nats": ("route_stats", _route_stats_natural_log),
    "stats-histogram-first-choice": ("route_stats", _route_stats_first_choice_only),
    "fp8-round-half-up": ("fp8_e4m3_encode", _fp8_round_half_up),
    "fp8-scale-full-range": ("quantize_rows_fp8", _quantize_full_range_scale),
    "bwd-silu-derivative-term-dropped": ("expert_ffn_backward", _expert_bwd_silu_prime_dropped),
    "bwd-gate-up-branches-swapped": ("expert_ffn_backward", _expert_bwd_branches_swapped),
    "bwd-softmax-sign": ("gates_backward", _gates_bwd_sign),
    "bwd-combine-without-gate": ("combine_backward", _combine_bwd_no_gate),
    "bwd-dispatch-first-copy-only": ("scatter_rows_backward", _scatter_bwd_first_row_only),
    "logits-fp32-accumulation": ("router_logits", _router_logits_fp32_accumulate),
    "logits-scaled-by-sqrt-d": ("router_logits", _router_logits_scaled),
    "bf16-bits-not-widened": ("_f64", _f64_without_widening),
    "bwd-swiglu-du-without-sigmoid": ("swiglu_backward", _swiglu_bwd_du_without_sigmoid),
    "fp8-weight-scale-per-column": ("quantize_weights_fp8", _fp8_weight_scale_per_column),
    "fp8-gemm-zero-point-dropped": ("gate_up_fp8", _gate_up_fp8_no_zero_point),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(om, attr, fn)
    caught = []
    for name, pin in PINS.items():
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(name)
    assert caught, f"no pin catches the planted mistake {mutant!r}"
