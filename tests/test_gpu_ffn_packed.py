"""Grouped SwiGLU FFN on packed expert weights: parity against the oracle on
the same bf16 inputs, on row tables that reach every number of live 32-row
token fragments of a tile (1..8), ragged tails, empty experts, K that is not a
multiple of the 128-wide k iteration, one rank's sub-table, and the whole
layer through moe_layer_fwd_packed."""
import numpy as np
import pytest
import torch

import oracle
from _gpu import TOL_LAYER, alloc, host, log, rel_err, upload
from test_gpu_ffn import _check, _weights
from top_routing_expert_amd import binding as B
from top_routing_expert_amd import configs as C
from top_routing_expert_amd import inputs as I

pytestmark = pytest.mark.gpu


def _run_packed(shape, x_perm, offs, wg, wu, wd):
    cfg = B.config(shape)
    A = x_perm.shape[0]
    pgu, pd = B.pack_weights(cfg, wg, wu, wd)
    h = torch.empty((A, shape.f), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((A, shape.d), dtype=torch.bfloat16, device="cuda")
    B.moe_ffn_gate_up_packed(cfg, x_perm, offs, pgu, h)
    B.moe_ffn_down_packed(cfg, h, offs, pd, y)
    torch.cuda.synchronize()
    return h, y


CASES = [
    # (E, d, f, counts)
    (8, 256, 448, [1, 33, 65, 97, 129, 161, 193, 225]),      # jn = 1..8
    (8, 320, 192, [129, 127, 1, 0, 300, 128, 256, 2]),      # K % 128 == 64 both ways
    (4, 128, 384, [256, 257, 512, 600]),                     # full tiles + tails
    (16, 128, 128, [0] * 7 + [517] + [0] * 8),               # one hot expert
    (4, 64, 64, [0, 0, 0, 1]),                               # one row
    (64, 128, 192, None),                                    # many small experts
    (8, 1024, 256, [40, 300, 0, 77, 256, 31, 5, 190]),      # long k loop (8 iterations)
]


@pytest.mark.parametrize("case", CASES, ids=[f"E{c[0]}-d{c[1]}-f{c[2]}" for c in CASES])
def test_packed_ffn_matches_oracle(case):
    E, d, f, counts = case
    log(f"[ffn-packed] {case[:3]}")
    rng = np.random.default_rng(E * d + f + 1)
    counts = rng.integers(0, 300, size=E) if counts is None else np.array(counts)
    A = int(counts.sum())
    shape = C.E8_D4096.replace(name="ffn-packed", T=A, k=1, E=E, d=d, f=f, ep_ranks=1)
    offs_np = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    xp_np = I.make_x(shape, seed=21)
    wg, wu, wd = _weights(shape, 22)
    dev = [B.to_device(a) for a in (xp_np, wg, wu, wd)]
    offs = torch.from_numpy(offs_np).cuda()
    h, y = _run_packed(shape, dev[0], offs, *dev[1:])
    _check(shape, xp_np, offs_np, wg, wu, wd, h, y)


def _counts_many(E):
    counts = np.zeros(E, dtype=np.int64)
    if E == 1024:  # mostly empty; live experts on both sides of 64-expert chunk edges
        for e, c in {0: 3, 63: 300, 64: 1, 65: 256, 127: 17, 128: 0, 500: 40, 1023: 5}.items():
            counts[e] = c
    elif E == 200:  # a partial last chunk and a run of empty experts across a chunk edge
        counts[:] = np.random.default_rng(200).integers(0, 40, size=E)
        counts[60:70] = 0
        counts[199] = 0
    else:  # 256 one-row experts and a large one
        counts[:] = 1
        counts[E - 1] = 600
    return counts


@pytest.mark.parametrize("E", [1024, 200, 256])
def test_packed_many_experts(E):
    """Layers of more than 16 experts find their tiles in a per-launch table of
    expert rows and first tiles: up to 1024 experts, empty runs on chunk
    edges, a partial last chunk, many one-row experts."""
    d, f = 128, 192
    counts = _counts_many(E)
    log(f"[ffn-packed] {E} experts, {int((counts > 0).sum())} with rows")
    A = int(counts.sum())
    shape = C.E8_D4096.replace(name="ffn-packed-many", T=A, k=1, E=E, d=d, f=f, ep_ranks=1)
    offs_np = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    xp_np = I.make_x(shape, seed=81)
    wg, wu, wd = _weights(shape, 82)
    dev = [B.to_device(a) for a in (xp_np, wg, wu, wd)]
    offs = torch.from_numpy(offs_np).cuda()
    h, y = _run_packed(shape, dev[0], offs, *dev[1:])
    _check(shape, xp_np, offs_np, wg, wu, wd, h, y)


# Problems with enough tiles to fill the chip run whole-slab tiles of up to
# 256 rows (the others half-slab tiles of up to 320 rows): these two shapes
# reach the whole-slab kernel for both GEMMs (E=64) and for the gate/up GEMM
# only (E=16), with experts above 256 rows, so both shapes and their ragged
# tails are covered.  Rows are sampled for the oracle.
WIDE = [
    (64, 2048, 1088, 0, 300),
    (16, 1024, 4096, 200, 700),
]


@pytest.mark.parametrize("case", WIDE, ids=[f"E{c[0]}-d{c[1]}-f{c[2]}" for c in WIDE])
def test_packed_ffn_whole_slab_tiles(case):
    E, d, f, lo, hi = case
    log(f"[ffn-packed] whole-slab tiles {case[:3]}")
    rng = np.random.default_rng(E + d + f)
    counts = rng.integers(lo, hi, size=E)
    counts[1] = 0
    A = int(counts.sum())
    shape = C.E8_D4096.replace(name="ffn-packed-wide", T=A, k=1, E=E, d=d, f=f, ep_ranks=1)
    offs_np = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    xp_np = I.make_x(shape, seed=71)
    wg, wu, wd = _weights(shape, 72)
    dev = [B.to_device(a) for a in (xp_np, wg, wu, wd)]
    offs = torch.from_numpy(offs_np).cuda()
    h, y = _run_packed(shape, dev[0], offs, *dev[1:])
    # every tile's first and last rows, plus a random sample
    rows = set(rng.choice(A, size=min(A, 384), replace=False).tolist())
    for e in range(E):
        r0, r1 = int(offs_np[e]), int(offs_np[e + 1])
        for r in range(r0, r1, 256):
            rows.update({r, min(r + 255, r1 - 1)})
    _check(shape, xp_np, offs_np, wg, wu, wd, h, y, rows=np.array(sorted(rows)))


def test_packed_matches_row_major_path():
    """Same sums in the same k order: the packed and row-major paths agree to
    within one bf16 rounding of h (identical in almost every element)."""
    log("[ffn-packed] vs row-major path")
    E, d, f = 8, 512, 320
    rng = np.random.default_rng(31)
    counts = rng.integers(0, 400, size=E)
    A = int(counts.sum())
    shape = C.E8_D4096.replace(name="ffn-packed-rm", T=A, k=1, E=E, d=d, f=f, ep_ranks=1)
    offs = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).cuda()
    xp = B.to_device(I.make_x(shape, seed=32))
    w = [B.to_device(a) for a in _weights(shape, 33)]
    h1, y1 = _run_packed(shape, xp, offs, *w)
    cfg = B.config(shape)
    h2 = torch.empty_like(h1)
    y2 = torch.empty_like(y1)
    B.moe_grouped_ffn(cfg, xp, offs, *w, h2, y2)
    torch.cuda.synchronize()
    hd = (h1.float() - h2.float()).abs()
    assert float(hd.max()) <= float(h2.float().abs().max()) * 2 ** -7
    assert float((hd > 0).float().mean()) < 0.01


def test_packed_subtable_runs_only_that_share():
    log("[ffn-packed] one rank's sub-table")
    E, R, d, f = 16, 4, 128, 192
    rng = np.random.default_rng(41)
    counts = rng.integers(1, 300, size=E)
    A = int(counts.sum())
    shape = C.E8_D4096.replace(name="ffn-packed-sub", T=A, k=1, E=E, d=d, f=f, ep_ranks=R)
    offs_np = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    xp_np = I.make_x(shape, seed=42)
    wg, wu, wd = _weights(shape, 43)
    xp, dg, du, dd = (B.to_device(a) for a in (xp_np, wg, wu, wd))
    offs = torch.from_numpy(offs_np).cuda()
    cfg = B.config(shape)
    pgu, pd = B.pack_weights(cfg, dg, du, dd)
    gu_bytes, d_bytes = B.packed_weight_bytes(cfg)
    per = E // R
    r = 1
    e0 = r * per
    sub = B.config(shape, E=per)
    hs = torch.full((A, f), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ys = torch.full((A, d), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    pgu_r = pgu[e0 * (gu_bytes // E):]
    pd_r = pd[e0 * (d_bytes // E):]
    B.moe_ffn_gate_up_packed(sub, xp, offs[e0:], pgu_r, hs)
    B.moe_ffn_down_packed(sub, hs, offs[e0:], pd_r, ys)
    torch.cuda.synchronize()
    r0, r1 = int(offs_np[e0]), int(offs_np[e0 + per])
    y_np, h_np = host(ys), host(hs)
    assert np.all(y_np[:r0] == 7) and np.all(y_np[r1:] == 7)
    assert np.all(h_np[:r0] == 7) and np.all(h_np[r1:] == 7)
    _check(shape, xp_np, offs_np, wg, wu, wd, hs, ys, rows=np.arange(r0, r1))


def test_packed_deterministic():
    log("[ffn-packed] determinism")
    E, d, f = 8, 256, 320
    rng = np.random.default_rng(51)
    counts = rng.integers(50, 300, size=E)
    A = int(counts.sum())
    shape = C.E8_D4096.replace(name="ffn-packed-det", T=A, k=1, E=E, d=d, f=f, ep_ranks=1)
    offs = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).cuda()
    xp = B.to_device(I.make_x(shape, seed=52))
    w = [B.to_device(a) for a in _weights(shape, 53)]
    h1, y1 = _run_packed(shape, xp, offs, *w)
    h2, y2 = _run_packed(shape, xp, offs, *w)
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("name", ["e8", "e64", "e16", "e256"])
def test_packed_layer_matches_oracle(name):
    """moe_layer_fwd_packed on the reduced workloads, against the oracle run on
    the GPU's own fp32 logits (so no routing flip can occur)."""
    shape = C.SMALL[name]
    log(f"[layer-packed] {shape.name}")
    inp = I.make_inputs(shape, seed=61)
    dev = upload(inp)
    buf = alloc(shape)
    cfg = B.config(shape)
    pgu, pd = B.pack_weights(cfg, dev["w_gate"], dev["w_up"], dev["w_down"])
    bufs = {k: buf[k] for k in ("logits", "topk_idx", "topk_w", "expert_offsets")}
    B.moe_layer_fwd_packed(cfg, dev["x"], dev["w_router"], dev["bias"], pgu, pd, buf["out"], bufs,
                           B.workspace(cfg, "layer"))
    torch.cuda.synchronize()
    ref = oracle.layer(inp["x"], inp["w_router"], inp["bias"], inp["w_gate"], inp["w_up"],
                       inp["w_down"], k=shape.k, n_group=shape.n_group,
                       topk_group=shape.topk_group, presel=shape.presel, renorm=shape.renorm,
                       ep_ranks=shape.ep_ranks, logits32=host(buf["logits"]))
    assert np.array_equal(host(buf["topk_idx"]), ref["topk_idx"])
    assert np.array_equal(host(buf["expert_offsets"]), ref["offsets"])
    err = rel_err(host(buf["out"]), ref["out"])
    assert err <= TOL_LAYER["bf16"], err


def _dispatch(shape, seed):
    """x in token order and the library's own dispatch of a random top-k."""
    rng = np.random.default_rng(seed)
    T, E, k = shape.T, shape.E, shape.k
    idx_np = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    cfg = B.config(shape)
    A = T * k
    x = B.to_device(I.make_x(shape, seed=seed + 1))
    idx = torch.from_numpy(idx_np).cuda()
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    roffs = torch.empty(shape.ep_ranks + 1, dtype=torch.int32, device="cuda")
    slot = torch.empty(A, dtype=torch.int32, device="cuda")
    src = torch.empty(A, dtype=torch.int32, device="cuda")
    xp = torch.empty((A, shape.d), dtype=torch.bfloat16, device="cuda")
    B.moe_permute(cfg, x, idx, offs, roffs, slot, src, xp, B.workspace(cfg, "permute"))
    return x, src, offs, xp


GATHER = [
    # (E, d, f, T, k): half-slab tiles of 1..10 fragments (2 x 2 pairs above 5),
    # and whole-slab tiles (E=64, f=1088)
    (8, 256, 448, 700, 2),
    (4, 320, 192, 333, 3),
    (64, 2048, 1088, 4000, 2),
]


@pytest.mark.parametrize("case", GATHER, ids=[f"E{c[0]}-d{c[1]}-f{c[2]}-T{c[3]}" for c in GATHER])
def test_packed_gather_equals_x_perm_path(case):
    """The gather reads x[src_of[p] / k] where the plain kernel reads x_perm[p]:
    same operands, same sums, so h is bit for bit the same."""
    E, d, f, T, k = case
    log(f"[ffn-packed] gather {case}")
    shape = C.E8_D4096.replace(name="ffn-gather", T=T, k=k, E=E, d=d, f=f, ep_ranks=1)
    x, src, offs, xp = _dispatch(shape, 81)
    cfg = B.config(shape)
    wg, wu, _ = _weights(shape, 82)
    pgu, _ = B.pack_weights(cfg, B.to_device(wg), B.to_device(wu), None)
    h1 = torch.empty((T * k, f), dtype=torch.bfloat16, device="cuda")
    h2 = torch.full((T * k, f), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    B.moe_ffn_gate_up_packed(cfg, xp, offs, pgu, h1)
    B.moe_ffn_gate_up_packed_gather(cfg, x, src, offs, pgu, h2)
    torch.cuda.synchronize()
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16))


def test_packed_gather_subtable():
    """One rank's experts: offsets and weights offset to the rank, src_of whole."""
    log("[ffn-packed] gather sub-table")
    E, R, d, f, T, k = 16, 4, 256, 320, 900, 2
    shape = C.E8_D4096.replace(name="ffn-gather-sub", T=T, k=k, E=E, d=d, f=f, ep_ranks=R)
    x, src, offs, xp = _dispatch(shape, 91)
    cfg = B.config(shape)
    wg, wu, _ = _weights(shape, 92)
    pgu, _ = B.pack_weights(cfg, B.to_device(wg), B.to_device(wu), None)
    gu_bytes, _ = B.packed_weight_bytes(cfg)
    per = E // R
    e0 = 2 * per
    sub = B.config(shape, E=per)
    h1 = torch.full((T * k, f), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    h2 = torch.full((T * k, f), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    B.moe_ffn_gate_up_packed(sub, xp, offs[e0:], pgu[e0 * (gu_bytes // E):], h1)
    B.moe_ffn_gate_up_packed_gather(sub, x, src, offs[e0:], pgu[e0 * (gu_bytes // E):], h2)
    torch.cuda.synchronize()
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16))
    r0, r1 = int(offs[e0]), int(offs[e0 + per])
    assert bool((h2[:r0].view(torch.int16) == 7).all()) and bool((h2[r1:].view(torch.int16) == 7).all())


def test_packed_layer_gather_equals_materialised():
    """moe_layer_fwd_packed with a caller x_perm (written and read) and without
    (gathered inside the first GEMM): the same out, bit for bit."""
    shape = C.SMALL["e64"]
    log(f"[layer-packed] gather vs x_perm {shape.name}")
    inp = I.make_inputs(shape, seed=63)
    dev = upload(inp)
    cfg = B.config(shape)
    pgu, pd = B.pack_weights(cfg, dev["w_gate"], dev["w_up"], dev["w_down"])
    outs = []
    for keep_xperm in (False, True):
        buf = alloc(shape)
        bufs = {"x_perm": buf["x_perm"]} if keep_xperm else {}
        B.moe_layer_fwd_packed(cfg, dev["x"], dev["w_router"], dev["bias"], pgu, pd, buf["out"],
                               bufs, B.workspace(cfg, "layer"))
        torch.cuda.synchronize()
        outs.append(buf["out"].view(torch.int16).clone())
    assert torch.equal(outs[0], outs[1])
