"""FP8 first GEMM: the FP8 weight image bit for bit against the oracle's
per-output-channel E4M3 quantisation, and h element by element against the
oracle's first GEMM on FP8 operands (gate_up_fp8), fed the GPU's own token
codes and the oracle's weight codes (shown equal to the image's).

Tolerance of h, from the arithmetic: the matrix instruction sums each
64-wide k block of code products to within 2^-11 of the block's largest
|product| (measured over every finite code pair), the blocks are added in
float32, the epilogue applies the scales and the centre's term in float32,
and h is rounded once to bf16 (relative 2^-8).  Against max(|h|, rms(h)) that
stays well below TOL_FP8 = 1e-2."""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

from _gpu import f64, host, log, rel_err
from oracle import moe_oracle as om
from top_routing_expert_amd import binding as B
from top_routing_expert_amd import configs as C
from top_routing_expert_amd import inputs as I

pytestmark = pytest.mark.gpu

TOL_FP8 = 1e-2


def _image_parts(shape, image):
    """(codes [E, 2f, d] uint8, scale [E, 2f], csum [E, 2f]) of an FP8 image
    laid out as include/moe.h states (parts 256-byte aligned)."""
    E, f, d = shape.E, shape.f, shape.d
    a256 = lambda n: (n + 255) // 256 * 256
    raw = host(image)
    n_codes = E * 2 * f * d
    scale_off = a256(n_codes)
    csum_off = scale_off + a256(E * 2 * f * 4)
    codes = raw[:n_codes].reshape(E, 2 * f, d)
    scale = raw[scale_off:scale_off + E * 2 * f * 4].view(np.float32).reshape(E, 2 * f)
    csum = raw[csum_off:csum_off + E * 2 * f * 4].view(np.float32).reshape(E, 2 * f)
    return codes, scale, csum


def _interleave_rows(f):
    """Packed row r -> (is_up, feature): per group of 16 features, 16 gate rows then 16 up rows."""
    r = np.arange(2 * f)
    return (r % 32) >= 16, 16 * (r // 32) + (r % 16)


def _check_image(shape, wg, wu, image, experts=None):
    codes, scale, csum = _image_parts(shape, image)
    is_up, feat = _interleave_rows(shape.f)
    for e in (range(shape.E) if experts is None else experts):
        gq, gs = om.quantize_weights_fp8(wg[e])
        uq, us = om.quantize_weights_fp8(wu[e])
        want_c = np.where(is_up[:, None], uq[feat], gq[feat])
        want_s = np.where(is_up, us[feat], gs[feat])
        assert np.array_equal(codes[e], want_c), e
        assert np.array_equal(scale[e].view(np.uint32), want_s.astype(np.float32).view(np.uint32)), e
        exact = om.fp8_e4m3_decode(want_c).sum(axis=1)  # exact in float64 (multiples of 2^-9)
        assert np.array_equal(csum[e].view(np.uint32), exact.astype(np.float32).view(np.uint32)), e


def _weights(shape, seed):
    return (I.make_expert_weight(shape, seed, I.TID_GATE), I.make_expert_weight(shape, seed, I.TID_UP))


@pytest.mark.parametrize("E,f,d", [(3, 64, 128), (8, 448, 256), (2, 192, 1024)])
def test_fp8_weight_image_bit_exact(E, f, d):
    shape = C.E8_D4096.replace(name="fp8-pack", T=16, E=E, f=f, d=d, ep_ranks=1)
    log(f"[fp8 gemm] pack E={E} f={f} d={d}")
    wg, wu = _weights(shape, 5)
    wg[0, 3] = 0  # an all-zero gate row: scale 0, codes 0
    image = B.pack_weights_fp8(B.config(shape), B.to_device(wg), B.to_device(wu))
    torch.cuda.synchronize()
    _check_image(shape, wg, wu, image)
    _, scale, _ = _image_parts(shape, image)
    assert scale[0, 2 * (3 // 16) * 16 + 3 % 16] == 0.0


def _run(shape, seed, counts=None):
    """Dispatch (indices), per-token FP8 codes, FP8 image, the FP8 first GEMM.
    Returns host copies of what the oracle needs."""
    rng = np.random.default_rng(seed)
    T, E, k = shape.T, shape.E, shape.k
    if counts is None:
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    else:  # k = 1: token t goes to the expert whose block holds t
        idx = np.repeat(np.arange(E), counts)[:, None].astype(np.int32)
    cfg = B.config(shape)
    x = I.make_x(shape, seed + 1)
    wg, wu = _weights(shape, seed + 2)
    dev_x = B.to_device(x)
    idx_d = torch.from_numpy(idx).cuda()
    A = T * k
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    roffs = torch.empty(shape.ep_ranks + 1, dtype=torch.int32, device="cuda")
    slot = torch.empty(A, dtype=torch.int32, device="cuda")
    src = torch.empty(A, dtype=torch.int32, device="cuda")
    B.moe_permute(cfg, None, idx_d, offs, roffs, slot, src, None, B.workspace(cfg, "permute"))
    codes = torch.empty((T, shape.d), dtype=torch.uint8, device="cuda")
    sz = torch.empty((T, 2), dtype=torch.float32, device="cuda")
    B.moe_quantize_fp8(cfg, dev_x, codes, sz)
    image = B.pack_weights_fp8(cfg, B.to_device(wg), B.to_device(wu))
    h = torch.full((A, shape.f), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    B.moe_ffn_gate_up_fp8_gather(cfg, codes, sz, src, offs, image, h)
    torch.cuda.synchronize()
    return dict(x=x, wg=wg, wu=wu, codes=host(codes), sz=host(sz), offs=host(offs),
                src=host(src), h=host(h), image=image)


def _oracle_h(shape, r, rows):
    """Oracle h of expert-ordered rows, expert by expert (on a few threads:
    numpy releases the GIL in its array work), on the GPU's token codes."""
    h = np.zeros((rows.size, shape.f))
    ex = np.searchsorted(r["offs"], rows, side="right") - 1
    experts = np.unique(ex)
    done = [0]

    def one(e):
        sel = np.flatnonzero(ex == e)
        t = r["src"][rows[sel]] // shape.k
        gq, gs = om.quantize_weights_fp8(r["wg"][e])
        uq, us = om.quantize_weights_fp8(r["wu"][e])
        h[sel], _, _ = om.gate_up_fp8(r["codes"][t], r["sz"][t, 0], r["sz"][t, 1], gq, gs, uq, us)
        done[0] += 1
        if done[0] % 32 == 0:
            log(f"    oracle: {done[0]} of {experts.size} experts")

    with cf.ThreadPoolExecutor(16) as pool:
        list(pool.map(one, experts))
    return h


CASES = [
    # (E, d, f, T, k): ragged tails of the 128-token tiles, many small
    # experts, experts of several row tiles with f not a multiple of 128
    (8, 256, 448, 700, 2),
    (64, 128, 192, 1500, 2),
    (16, 512, 1088, 2048, 2),
    # many experts over several 64-expert chunks, most with a few rows or none
    (512, 128, 128, 600, 4),
]


@pytest.mark.parametrize("case", CASES, ids=[f"E{c[0]}-d{c[1]}-f{c[2]}-T{c[3]}" for c in CASES])
def test_gate_up_fp8_matches_oracle(case):
    E, d, f, T, k = case
    shape = C.E8_D4096.replace(name="fp8-gemm", T=T, k=k, E=E, d=d, f=f, ep_ranks=1)
    log(f"[fp8 gemm] {case}")
    r = _run(shape, 11 + E)
    rows = np.arange(T * k)
    err = rel_err(r["h"], _oracle_h(shape, r, rows))
    log(f"  h err={err:.3e}")
    assert err <= TOL_FP8


@pytest.mark.parametrize("kind", ["one-expert", "single-rows", "empty-and-ragged"])
def test_gate_up_fp8_edge_row_tables(kind):
    E, d, f = 8, 256, 320
    counts = {"one-expert": [0, 0, 0, 517, 0, 0, 0, 0],
              "single-rows": [1, 1, 1, 1, 1, 1, 1, 1],
              "empty-and-ragged": [129, 0, 1, 300, 0, 257, 33, 2]}[kind]
    T = int(sum(counts))
    shape = C.E8_D4096.replace(name="fp8-edge", T=T, k=1, E=E, d=d, f=f, ep_ranks=1)
    log(f"[fp8 gemm] {kind}")
    r = _run(shape, 21, counts=np.array(counts))
    assert np.array_equal(np.diff(r["offs"]), counts)
    err = rel_err(r["h"], _oracle_h(shape, r, np.arange(T)))
    log(f"  h err={err:.3e}")
    assert err <= TOL_FP8


def test_gate_up_fp8_empty_batch():
    shape = C.E8_D4096.replace(name="fp8-empty", T=0, d=256, f=128)
    cfg = B.config(shape)
    B.moe_ffn_gate_up_fp8_gather(cfg, None, None, None, None, None, None)
    torch.cuda.synchronize()


@pytest.mark.parametrize("ci", [2, 5])
def test_gate_up_fp8_full_size_sampled(ci):
    """The T1024-d4096-E8 and T8192-d7168-E256 workloads on their own routing:
    the weight image of a few experts bit for bit, h on the first and last row
    of every 128- and 256-row tile of the checked experts plus a random
    sample of their rows."""
    shape = C.CONFIGS[ci - 1]
    log(f"[fp8 gemm] full {shape.name}: inputs")
    inp = I.make_inputs(shape, seed=ci)
    cfg = B.config(shape)
    dev = {n: B.to_device(inp[n]) for n in ("x", "w_router", "w_gate", "w_up")}
    bias = None if inp["bias"] is None else B.to_device(inp["bias"])
    T, E, k, d, f = shape.T, shape.E, shape.k, shape.d, shape.f
    A = T * k
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    B.moe_route(cfg, dev["x"], dev["w_router"], bias, logits, idx, w, B.workspace(cfg, "route"))
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    roffs = torch.empty(shape.ep_ranks + 1, dtype=torch.int32, device="cuda")
    slot = torch.empty(A, dtype=torch.int32, device="cuda")
    src = torch.empty(A, dtype=torch.int32, device="cuda")
    B.moe_permute(cfg, None, idx, offs, roffs, slot, src, None, B.workspace(cfg, "permute"))
    codes = torch.empty((T, d), dtype=torch.uint8, device="cuda")
    sz = torch.empty((T, 2), dtype=torch.float32, device="cuda")
    B.moe_quantize_fp8(cfg, dev["x"], codes, sz)
    image = B.pack_weights_fp8(cfg, dev["w_gate"], dev["w_up"])
    del dev
    h = torch.empty((A, f), dtype=torch.bfloat16, device="cuda")
    B.moe_ffn_gate_up_fp8_gather(cfg, codes, sz, src, offs, image, h)
    torch.cuda.synchronize()
    log("  image of three experts")
    _check_image(shape, inp["w_gate"], inp["w_up"], image, experts=[0, E // 2, E - 1])
    r = dict(wg=inp["w_gate"], wu=inp["w_up"], codes=host(codes), sz=host(sz), offs=host(offs),
             src=host(src), h=host(h))
    # every expert of the E = 8 layer; 64 evenly spaced experts of the E = 256
    # one (the oracle quantises each checked expert's 30 M weights on the CPU)
    rng = np.random.default_rng(ci)
    o = r["offs"].astype(np.int64)
    rows = set()
    for e in np.unique(np.linspace(0, E - 1, min(E, 64)).astype(int)):
        c = int(o[e + 1] - o[e])
        if c == 0:
            continue
        rows.update(rng.integers(o[e], o[e + 1], size=min(c, 8)).tolist())
        for tm in (128, 256):
            mt = -(-c // tm)
            for m in range(mt):
                rows.update((int(o[e]) + m * c // mt, int(o[e]) + (m + 1) * c // mt - 1))
    rows = np.array(sorted(x for x in rows if 0 <= x < A))
    log(f"  oracle h on {rows.size} rows")
    err = rel_err(r["h"][rows], _oracle_h(shape, r, rows))
    log(f"  h err={err:.3e}")
    assert err <= TOL_FP8


def test_fp8_layer_matches_oracle():
    """The whole layer with the FP8 first GEMM (route, index-only dispatch,
    per-token FP8 codes, FP8 gate/up, bf16 down projection, combine) against
    the oracle's composition of the same steps on the same routing."""
    shape = C.SMALL["e8"]
    log(f"[fp8 gemm] layer {shape.name}")
    inp = I.make_inputs(shape, seed=41)
    cfg = B.config(shape)
    dev = {n: (None if v is None else B.to_device(v)) for n, v in inp.items()}
    T, E, k, d, f = shape.T, shape.E, shape.k, shape.d, shape.f
    A = T * k
    bufs = {n: torch.empty(s, dtype=t, device="cuda") for n, s, t in (
        ("logits", (T, E), torch.float32), ("idx", (T, k), torch.int32),
        ("w", (T, k), torch.float32), ("offs", (E + 1,), torch.int32),
        ("roffs", (shape.ep_ranks + 1,), torch.int32), ("slot", (A,), torch.int32),
        ("src", (A,), torch.int32), ("codes", (T, d), torch.uint8), ("sz", (T, 2), torch.float32),
        ("h", (A, f), torch.bfloat16), ("y", (A, d), torch.bfloat16),
        ("out", (T, d), torch.bfloat16))}
    b = bufs
    B.moe_route(cfg, dev["x"], dev["w_router"], dev["bias"], b["logits"], b["idx"], b["w"],
                B.workspace(cfg, "route"))
    B.moe_permute(cfg, None, b["idx"], b["offs"], b["roffs"], b["slot"], b["src"], None,
                  B.workspace(cfg, "permute"))
    B.moe_quantize_fp8(cfg, dev["x"], b["codes"], b["sz"])
    image = B.pack_weights_fp8(cfg, dev["w_gate"], dev["w_up"])
    _, pd = B.pack_weights(cfg, None, None, dev["w_down"])
    B.moe_ffn_gate_up_fp8_gather(cfg, b["codes"], b["sz"], b["src"], b["offs"], image, b["h"])
    B.moe_ffn_down_packed(cfg, b["h"], b["offs"], pd, b["y"])
    B.moe_combine(cfg, b["y"], b["slot"], b["w"], b["out"])
    torch.cuda.synchronize()
    idx = host(b["idx"])
    r_idx, r_w, _ = om.route(host(b["logits"]), inp["bias"], k=k, n_group=shape.n_group,
                             topk_group=shape.topk_group, presel=shape.presel,
                             renorm=shape.renorm)
    assert np.array_equal(idx, r_idx)
    p = om.permute(idx, E, shape.ep_ranks)
    r = dict(wg=inp["w_gate"], wu=inp["w_up"], codes=host(b["codes"]), sz=host(b["sz"]),
             offs=p["offsets"], src=p["src_of"])
    h_ref = _oracle_h(shape, r, np.arange(A))
    y_ref = np.zeros((A, d))
    for e in range(E):
        r0, r1 = int(p["offsets"][e]), int(p["offsets"][e + 1])
        y_ref[r0:r1] = h_ref[r0:r1] @ f64(inp["w_down"][e]).T
    out_ref = om.combine(y_ref, p["slot_of"], r_w)
    err = rel_err(host(b["out"]), out_ref)
    log(f"  out err={err:.3e}")
    assert err <= 2e-2
