"""Router parity: HIP path (through the C ABI) vs the CPU oracle.

Selection must be bit-exact given identical fp32 logits; gates within
GATE_TOL; the GPU's fp32 logits within the worst-case fp32 summation bound of
the oracle's fp64 logits."""
import numpy as np
import pytest
import torch

from _gpu import (GATE_TOL, FLIP_MARGIN, alloc, host, log, logits_bound, routing_kwargs,
                  upload)
from oracle import moe_oracle as om
from top_routing_expert_amd import binding as B
from top_routing_expert_amd import configs as C
from top_routing_expert_amd import inputs as I

pytestmark = pytest.mark.gpu


def _route(shape, dev, buf):
    cfg = B.config(shape)
    B.moe_route(cfg, dev["x"], dev["w_router"], dev["bias"], buf["logits"], buf["topk_idx"],
                buf["topk_w"], B.workspace(cfg, "route"))
    torch.cuda.synchronize()


def _check_route(shape, inp, buf, rows_for_bound=None):
    z = host(buf["logits"])
    idx = host(buf["topk_idx"])
    w = host(buf["topk_w"])
    rows = rows_for_bound if rows_for_bound is not None else np.arange(shape.T)
    z64 = om.router_logits(inp["x"][rows], inp["w_router"])
    assert np.all(np.abs(z[rows] - z64) <= logits_bound(inp["x"], inp["w_router"], rows))
    o_idx, o_w, _ = om.route(z, inp["bias"], **routing_kwargs(shape))
    bad = np.flatnonzero(np.any(idx != o_idx, axis=1))
    assert bad.size == 0, f"{bad.size} tokens differ, first {bad[:5]}: {idx[bad[:3]]} vs {o_idx[bad[:3]]}"
    assert np.max(np.abs(w - o_w)) <= GATE_TOL
    return z, idx


# expert counts whose gate GEMM takes the 32-, 128- and 256-wide expert blocks
# (the workloads only reach the E <= 16, 64 and 256 shapes), with ragged T and E
GEMM_SHAPES = [dict(E=24, k=2, T=333, d=320), dict(E=100, k=5, T=257, d=256, presel=20),
               dict(E=1024, k=16, T=130, d=128, n_group=64, topk_group=16, presel=32)]


@pytest.mark.parametrize("over", GEMM_SHAPES, ids=[str(o) for o in GEMM_SHAPES])
def test_route_gemm_expert_blocks(over):
    shape = C.E8_D4096.replace(name="route-blocks", ep_ranks=1, renorm=1, **over)
    log(f"[route] gate GEMM blocks {over}")
    inp = I.make_inputs(shape, seed=23, with_experts=False)
    dev, buf = upload(inp), alloc(shape)
    _route(shape, dev, buf)
    _check_route(shape, inp, buf)


# The E <= 16 stream over x: one k-pair, a split count that does not divide
# d's k-pairs, many splits of short k ranges, and a very wide d (1152 k-pairs
# over 16 splits) with a handful of tokens
SKINNY_SHAPES = [dict(E=8, k=2, T=70, d=64), dict(E=16, k=2, T=333, d=4160),
                 dict(E=6, k=2, T=1500, d=2048), dict(E=8, k=2, T=5, d=73728)]


@pytest.mark.parametrize("over", SKINNY_SHAPES, ids=[str(o) for o in SKINNY_SHAPES])
def test_route_skinny_shapes(over):
    shape = C.E8_D4096.replace(name="route-skinny", ep_ranks=1, renorm=1, **over)
    log(f"[route] E <= 16 stream {over}")
    inp = I.make_inputs(shape, seed=29, with_experts=False)
    dev, buf = upload(inp), alloc(shape)
    _route(shape, dev, buf)
    _check_route(shape, inp, buf)


# E <= 16 routers on short batches: one token, a ragged last block of tokens,
# wide and narrow d, bias without renormalisation, every lane count of the
# selection
SMALL_BATCH_SHAPES = [dict(E=8, k=2, T=1, d=512), dict(E=3, k=2, T=7, d=1024),
                      dict(E=16, k=2, T=2048, d=4096), dict(E=12, k=3, T=333, d=3584, renorm=0, bias="normal"),
                      dict(E=2, k=1, T=64, d=1536), dict(E=5, k=4, T=1030, d=2560)]


@pytest.mark.parametrize("over", SMALL_BATCH_SHAPES, ids=[str(o) for o in SMALL_BATCH_SHAPES])
def test_route_short_batches(over):
    over = dict(over)
    shape = C.E8_D4096.replace(name="route-small", ep_ranks=1, **{"renorm": 1, **over})
    log(f"[route] short batch {over}")
    inp = I.make_inputs(shape, seed=31, with_experts=False)
    dev, buf = upload(inp), alloc(shape)
    _route(shape, dev, buf)
    _check_route(shape, inp, buf)


@pytest.mark.parametrize("key", list(C.SMALL), ids=list(C.SMALL))
def test_route_small_shapes(key):
    shape = C.SMALL[key]
    log(f"[route] small {shape.name}")
    inp = I.make_inputs(shape, seed=21, with_experts=False)
    dev, buf = upload(inp), alloc(shape)
    _route(shape, dev, buf)
    _check_route(shape, inp, buf)


@pytest.mark.parametrize("shape", C.CONFIGS, ids=lambda s: s.name)
def test_route_full_size(shape):
    log(f"[route] full {shape.name}")
    inp = I.make_inputs(shape, seed=shape.E + 1, with_experts=False)
    dev, buf = upload(inp), alloc(shape)
    _route(shape, dev, buf)
    rows = np.random.default_rng(0).choice(shape.T, size=min(shape.T, 512), replace=False)
    z, idx = _check_route(shape, inp, buf, rows)
    # informational: disagreement with the oracle's own fp64 logits happens
    # only at near-ties
    s64 = om.router_logits(inp["x"], inp["w_router"])
    if inp["bias"] is not None:
        s64 = s64 + inp["bias"].astype(np.float64)[None, :]
    o_idx, _, _ = om.route(s64.astype(np.float32), None, **routing_kwargs(shape))
    flips = np.flatnonzero(np.any(np.sort(idx, 1) != np.sort(o_idx, 1), axis=1))
    margin = om.margins(s64, shape.k, shape.n_group, shape.topk_group)
    assert np.all(margin[flips] < FLIP_MARGIN)
    log(f"  flips vs fp64 logits: {flips.size}")


ROUTING_CASES = [
    dict(E=8, k=2),
    dict(E=8, k=2, bias=True),
    dict(E=64, k=2, presel=8, renorm=0, bias=True),
    dict(E=16, k=2),
    dict(E=256, k=8, n_group=8, topk_group=4),
    dict(E=1024, k=16, presel=32, n_group=64, topk_group=16),
    dict(E=3, k=3),
    dict(E=1, k=1),
    dict(E=12, k=3, renorm=0),
    dict(E=100, k=5, presel=20, renorm=1),
    dict(E=32, k=4, n_group=32, topk_group=4),
    # 64 < E <= 256 runs 32 lanes per token when n_group <= 32, else 64
    dict(E=128, k=6, n_group=32, topk_group=8),
    dict(E=192, k=8, n_group=64, topk_group=16),
]


@pytest.mark.parametrize("case", ROUTING_CASES, ids=[str(c) for c in ROUTING_CASES])
@pytest.mark.parametrize("T", [1, 777])
def test_selection_on_given_logits_with_ties(case, T):
    """x = NULL: the logits are an input; exact ties, +-0 and bias are common."""
    case = dict(case)
    use_bias = case.pop("bias", False)
    fields = dict(name="given-logits", T=T, d=64, f=64, ep_ranks=1, n_group=1, topk_group=1,
                  presel=0, renorm=1)
    fields.update(case)
    shape = C.E8_D4096.replace(**fields)
    log(f"[route] given logits T={T} {case} bias={use_bias}")
    rng = np.random.default_rng(T * 1000 + shape.E)
    z = (rng.integers(-3, 4, size=(T, shape.E)) * 0.5).astype(np.float32)
    z[rng.random((T, shape.E)) < 0.1] = -0.0
    bias = None
    if use_bias:
        bias = (rng.integers(-2, 3, size=shape.E) * 0.5).astype(np.float32)
        bias[0] = -0.0
    logits = torch.from_numpy(z).cuda()
    bias_d = None if bias is None else torch.from_numpy(bias).cuda()
    idx = torch.empty((T, shape.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, shape.k), dtype=torch.float32, device="cuda")
    B.moe_route(B.config(shape), None, None, bias_d, logits, idx, w, None)
    torch.cuda.synchronize()
    o_idx, o_w, _ = om.route(z, bias, **routing_kwargs(shape))
    assert np.array_equal(host(idx), o_idx)
    assert np.max(np.abs(host(w) - o_w)) <= GATE_TOL
    assert np.array_equal(host(logits), z)  # an input stays untouched


def test_route_empty_batch():
    log("[route] T=0")
    shape = C.E8_D4096.replace(T=0)
    cfg = B.config(shape)
    B.moe_route(cfg, None, None, None, None, None, None, None)
    torch.cuda.synchronize()
