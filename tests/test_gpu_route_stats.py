"""Routing diagnostics (moe_route_stats) against the oracle on the library's
own route and dispatch outputs: histogram and per-rank load bit-exact, the
four float statistics within STATS_TOL (fp32 exp / log2 and fixed-order fp32
sums on the GPU, float64 in the oracle)."""
import numpy as np
import pytest
import torch

from _gpu import alloc, host, log, upload
from oracle import moe_oracle as om
from top_routing_expert_amd import binding as B
from top_routing_expert_amd import configs as C
from top_routing_expert_amd import inputs as I

pytestmark = pytest.mark.gpu

# fp32 softmax / entropy terms of magnitude <= log2 E, summed over <= 2^14
# tokens in fp32: relative error ~ a few 1e-6; 2e-4 leaves a wide margin
STATS_TOL = 2e-4


def _stats(shape, seed):
    inp = I.make_inputs(shape, seed=seed)
    dev = upload(inp)
    buf = alloc(shape)
    cfg = B.config(shape)
    B.moe_route(cfg, dev["x"], dev["w_router"], dev["bias"], buf["logits"], buf["topk_idx"],
                buf["topk_w"], B.workspace(cfg, "route"))
    B.moe_permute(cfg, None, buf["topk_idx"], buf["expert_offsets"], buf["rank_offsets"],
                  buf["slot_of"], buf["src_of"], None, B.workspace(cfg, "permute"))
    hist = torch.full((shape.E,), -7, dtype=torch.int32, device="cuda")
    rload = torch.full((shape.ep_ranks,), -7, dtype=torch.int32, device="cuda")
    stats = torch.full((4,), -7.0, dtype=torch.float32, device="cuda")
    B.moe_route_stats(cfg, buf["logits"], dev["bias"], buf["expert_offsets"], buf["rank_offsets"],
                      hist, rload, stats, B.workspace(cfg, "route_stats"))
    torch.cuda.synchronize()
    ref = om.route_stats(host(buf["logits"]), inp["bias"], host(buf["topk_idx"]), shape.E,
                         shape.ep_ranks, shape.presel)
    return host(hist), host(rload), host(stats), ref


def _check(hist, rload, stats, ref):
    assert np.array_equal(hist, ref["hist"])
    assert np.array_equal(rload, ref["rank_load"])
    want = [ref["token_entropy_bits"], ref["presel_gap"], ref["load_entropy_bits"],
            ref["max_load_ratio"]]
    for got, w in zip(stats.tolist(), want):
        assert abs(got - w) <= STATS_TOL * max(1.0, abs(w)), (stats.tolist(), want)


@pytest.mark.parametrize("key", list(C.SMALL), ids=list(C.SMALL))
def test_route_stats_small_shapes(key):
    shape = C.SMALL[key]
    log(f"[route-stats] {shape.name}")
    _check(*_stats(shape, 101))


def test_route_stats_many_experts():
    """1024 experts (16 scores per lane), pre-selection and groups."""
    shape = C.SMALL["e64"].replace(name="stats-e1024", T=300, E=1024, k=16, presel=32, renorm=0,
                                   n_group=64, topk_group=16, ep_ranks=16, d=128)
    log(f"[route-stats] {shape.name}")
    _check(*_stats(shape, 103))


@pytest.mark.parametrize("shape", C.CONFIGS, ids=lambda s: s.name)
def test_route_stats_full_size(shape):
    log(f"[route-stats] {shape.name}")
    hist, rload, stats, ref = _stats(shape, C.CONFIGS.index(shape) + 1)
    _check(hist, rload, stats, ref)
    assert hist.sum() == shape.T * shape.k


def test_route_stats_deterministic_and_empty():
    shape = C.SMALL["e64"]
    log("[route-stats] determinism, T = 0")
    a = _stats(shape, 7)[2]
    b = _stats(shape, 7)[2]
    assert np.array_equal(a.view(np.int32), b.view(np.int32))
    empty = shape.replace(T=0)
    cfg = B.config(empty)
    hist = torch.full((empty.E,), -7, dtype=torch.int32, device="cuda")
    rload = torch.full((empty.ep_ranks,), -7, dtype=torch.int32, device="cuda")
    stats = torch.full((4,), -7.0, dtype=torch.float32, device="cuda")
    B.moe_route_stats(cfg, None, None, None, None, hist, rload, stats, None)
    torch.cuda.synchronize()
    assert not host(hist).any() and not host(rload).any() and not host(stats).any()
