"""Expert waves (moe_layer_fwd_packed_waved): every output bit for bit equal
to the serial layer (moe_layer_fwd_packed with the gather in the first
GEMM), for several wave counts, with the waves split over two streams or on
one, on the reduced workloads and at full size."""
import numpy as np
import pytest
import torch

from _gpu import alloc, host, log, upload
from top_routing_expert_amd import binding as B
from top_routing_expert_amd import configs as C
from top_routing_expert_amd import inputs as I

pytestmark = pytest.mark.gpu

FIELDS = ("logits", "topk_idx", "topk_w", "expert_offsets", "rank_offsets", "slot_of", "src_of",
          "h", "y_perm")


def _bufs(buf):
    return {n: buf[n] for n in FIELDS}


def _bits(t):
    return host(t).view(np.uint8)


def _compare(shape, inp, waves_list, two_streams=True):
    cfg = B.config(shape)
    dev = upload(inp)
    pgu, pd = B.pack_weights(cfg, dev["w_gate"], dev["w_up"], dev["w_down"])
    ws = B.workspace(cfg, "layer")
    ref = alloc(shape)
    B.moe_layer_fwd_packed(cfg, dev["x"], dev["w_router"], dev["bias"], pgu, pd, ref["out"],
                           _bufs(ref), ws)
    torch.cuda.synchronize()
    want = {n: _bits(ref[n]) for n in FIELDS + ("out",)}
    aux = torch.cuda.Stream() if two_streams else None  # default priority
    for W in waves_list:
        got = alloc(shape)
        for t in got.values():  # stale values must all be overwritten
            t.view(torch.uint8).fill_(0x5A)
        ws2 = B.workspace(cfg, "layer")
        B.moe_layer_fwd_packed_waved(cfg, dev["x"], dev["w_router"], dev["bias"], pgu, pd,
                                     got["out"], _bufs(got), ws2, n_waves=W, aux_stream=aux)
        torch.cuda.synchronize()
        for n in FIELDS + ("out",):
            assert np.array_equal(_bits(got[n]), want[n]), (W, n)
        log(f"  {shape.name}: {W} waves ({'two streams' if aux is not None else 'one stream'}) "
            "bit for bit")


@pytest.mark.parametrize("key,waves", [("e8", (1, 2, 4, 8)), ("e64", (2, 8, 64)),
                                       ("e16", (2, 4)), ("e256", (2, 4, 8, 32))])
def test_waves_equal_serial_small(key, waves):
    shape = C.SMALL[key]
    log(f"[waves] {shape.name}")
    _compare(shape, I.make_inputs(shape, seed=51), waves)


def test_waves_on_one_stream():
    shape = C.SMALL["e256"]
    log(f"[waves] {shape.name} on one stream")
    _compare(shape, I.make_inputs(shape, seed=52), (4,), two_streams=False)


def test_waves_single_token_and_empty_waves():
    """One token: at most k experts hold rows, so most waves have no rows at
    all and combine no token."""
    shape = C.SMALL["e64"].replace(name="waves-T1", T=1)
    log(f"[waves] {shape.name}")
    _compare(shape, I.make_inputs(shape, seed=53), (8, 64))


@pytest.mark.parametrize("ci,waves", [(2, (2, 4)), (5, (2, 4, 8))])
def test_waves_equal_serial_full_size(ci, waves):
    shape = C.CONFIGS[ci - 1]
    log(f"[waves] full {shape.name}")
    _compare(shape, I.make_inputs(shape, seed=ci), waves)


def test_waves_empty_batch():
    shape = C.SMALL["e8"].replace(name="waves-T0", T=0)
    cfg = B.config(shape)
    B.moe_layer_fwd_packed_waved(cfg, None, None, None, None, None, None, None,
                                 B.workspace(cfg, "layer"), n_waves=2)
    torch.cuda.synchronize()
