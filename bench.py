#!/usr/bin/env python3
"""MoE-layer forward throughput on one MI355X.

One step = one pass of the whole path over one batch of synthetic tokens:
moe_route -> moe_permute -> moe_ffn_gate_up -> moe_ffn_down -> moe_combine,
each a C-ABI call that enqueues the HIP kernels on the current stream.  With
the packed FFN the dispatch's row gather runs inside the first GEMM by default
(moe_permute writes the indices, moe_ffn_gate_up_packed_gather reads the token
rows through src_of); --dispatch copy materialises x_perm first.
Inputs are resident in HBM before timing starts.  W warm-up steps, then K
timed steps bracketed by device synchronisation; one pair of HIP events on
the library's stream brackets the dominant kernel in every timed step.
Prints ONE JSON line.

Default workload (the line's `value`): T=8192 tokens, d=7168, E=256 experts
in 8 groups of 32 with the best 4 groups kept, top-8, SwiGLU f=2048, bf16 --
the largest of the five workloads.  The four others (the fp32 tiny layer, the
E=8, E=64 and E=16 layers) are run after it, each timed the same way, and
reported under "workloads", and the FP8 first GEMM and the expert waves
are timed on the default workload under "variants".

`forward_calls` is the one definition of the timed call sequence; the
full-size parity tests run the same function.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0     # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3   # MI355X fp32 vector
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA
PHASES = ("route", "permute", "ffn_gate_up", "ffn_down", "combine")
DOMINANT = "ffn_gate_up"
FLIP_MARGIN = 1e-4
HEADLINE = 5
CSRC = os.path.join(ROOT, "top_routing_expert_amd", "csrc")
# per FFN weight layout: (counter summary, kernel sources it was taken on, kernel name)
FFN_KERNELS = {
    "rowmajor": (os.path.join(ROOT, "profiles", "ffn_gate_up_traffic.json"),
                 [os.path.join(CSRC, n) for n in ("ffn.hip", "tiles.h", "common.h")],
                 "grouped_gemm_bf16_kernel<gated> (moe_ffn_gate_up)"),
    "packed": (os.path.join(ROOT, "profiles", "ffn_gate_up_packed_traffic.json"),
               [os.path.join(CSRC, n) for n in ("ffn_packed.hip", "tiles.h", "common.h")],
               "grouped_gemm_packed_kernel<gated> (moe_ffn_gate_up_packed)"),
}


def kernel_sources_sha256(paths):
    """One hash over the kernel's source files (in the given order)."""
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def shape_of(spec):
    from top_routing_expert_amd import configs as C
    spec = str(spec)
    return C.CONFIGS[int(spec) - 1] if spec.isdigit() else C.BY_NAME[spec]


def seed_of(shape):
    from top_routing_expert_amd import configs as C
    return C.CONFIGS.index(shape) + 1 if shape in C.CONFIGS else 1


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=str(HEADLINE),
                    help="workload of the line's value: index 1..5 or name; default 5 "
                         "(T8192-d7168-E256-g8x4-top8-f2048)")
    ap.add_argument("--also", default="auto",
                    help="other workloads timed after it, comma-separated indices or names; "
                         "'auto' = the four others when the default workload is timed, "
                         "'none' = no others")
    ap.add_argument("--cpu-tokens", type=int, default=256,
                    help="tokens of the workload the CPU oracle baseline runs (0 = skip)")
    ap.add_argument("--ffn", choices=sorted(FFN_KERNELS), default="packed",
                    help="expert-weight layout of the grouped FFN: packed once at load time "
                         "(moe_pack_weights) or the plain [E,f,d] / [E,d,f] arrays")
    ap.add_argument("--dispatch", choices=("gather", "copy", "fp8", "fp8gemm"), default="gather",
                    help="packed FFN: gather the token rows inside the first GEMM (the dispatch "
                         "writes indices only), copy them to x_perm first, send them as "
                         "per-token FP8 (quantize, then decode into x_perm in expert order), or "
                         "feed the per-token FP8 codes to an FP8 first GEMM on E4M3 weights "
                         "(fp8gemm; the down projection stays bf16)")
    ap.add_argument("--diagnostics", action="store_true",
                    help="also time the routing diagnostics (moe_route_stats) after the dispatch; "
                         "reported as its own phase and included in the step")
    ap.add_argument("--backward", action="store_true",
                    help="time forward + backward (combine, grouped FFN, router and dispatch "
                         "backward on the forward's routing) instead of the forward alone")
    ap.add_argument("--no-flush-pass", action="store_true",
                    help="skip the extra pass that evicts the 256 MB MALL before every step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for counter calibration)")
    ap.add_argument("--variants", default="auto", choices=("auto", "none", "all"),
                    help="also time, on the line's workload, the FP8 first GEMM path and the "
                         "expert waves (reported under \"variants\"); 'auto' = with the default "
                         "line only")
    a = ap.parse_args(argv)
    a.shape = shape_of(a.config)
    default_line = not (a.config != str(HEADLINE) or a.backward or a.diagnostics
                        or a.dispatch != "gather" or a.ffn != "packed")
    if a.variants == "auto":
        a.variants = "all" if default_line else "none"
    if a.also == "auto":
        a.also = "1,2,3,4" if default_line else "none"
    a.others = [] if a.also == "none" else [shape_of(s) for s in a.also.split(",") if s]
    return a


# ----------------------------------------------------------------------------- the path
def modes_for(shape, ffn="packed", dispatch="gather", backward=False):
    """The layout and dispatch a workload actually runs with: packed images are
    bf16 only, the gather is a packed-FFN kernel, the backward reads x_perm."""
    if shape.dtype != "bf16":
        ffn = "rowmajor"
    if ffn != "packed" or backward:
        dispatch = "copy"
    return ffn, dispatch


def prepare(shape, inp, ffn="packed", dispatch="gather", backward=False, keep_plain=False):
    """Device inputs, output buffers, workspaces and (for the packed layout)
    the expert weights packed once, as a model does at load time."""
    import torch
    from top_routing_expert_amd import binding as B

    ffn, dispatch = modes_for(shape, ffn, dispatch, backward)
    dev = {k: (None if v is None else B.to_device(v)) for k, v in inp.items()}
    cfg = B.config(shape)
    T, E, k, d, f, R = shape.T, shape.E, shape.k, shape.d, shape.f, shape.ep_ranks
    A = T * k
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    gather, fp8 = dispatch == "gather", dispatch in ("fp8", "fp8gemm")
    fp8gemm = dispatch == "fp8gemm"
    e = lambda *s, t=dt: torch.empty(s, dtype=t, device="cuda")
    buf = dict(
        logits=e(T, E, t=torch.float32), topk_idx=e(T, k, t=torch.int32),
        topk_w=e(T, k, t=torch.float32), expert_offsets=e(E + 1, t=torch.int32),
        rank_offsets=e(R + 1, t=torch.int32), slot_of=e(A, t=torch.int32),
        src_of=e(A, t=torch.int32), x_perm=None if (gather or fp8gemm) else e(A, d),
        codes=e(T, d, t=torch.uint8) if fp8 else None,
        scale_zero=e(T, 2, t=torch.float32) if fp8 else None,
        h=e(A, f), y_perm=e(A, d), out=e(T, d))
    ctx = dict(shape=shape, cfg=cfg, dev=dev, buf=buf, ffn=ffn, dispatch=dispatch,
               backward=backward, ws_route=B.workspace(cfg, "route"),
               ws_permute=B.workspace(cfg, "permute"), packed=None)
    if ffn == "packed":
        log("packing expert weights")
        if fp8gemm:  # E4M3 gate/up image; the down projection keeps its bf16 image
            ctx["fp8_image"] = B.pack_weights_fp8(cfg, dev["w_gate"], dev["w_up"])
            ctx["packed"] = B.pack_weights(cfg, None, None, dev["w_down"])
        else:
            ctx["packed"] = B.pack_weights(cfg, dev["w_gate"], dev["w_up"], dev["w_down"])
        torch.cuda.synchronize()
        if not (backward or keep_plain):  # the plain arrays are then dropped
            dev["w_gate"] = dev["w_up"] = dev["w_down"] = None
    return ctx


def forward_calls(ctx, stream=None):
    """The forward as timed: an ordered {phase: call} of C-ABI calls that
    enqueue on `stream` (default: torch's current stream)."""
    import torch
    from top_routing_expert_amd import binding as B

    stream = torch.cuda.current_stream() if stream is None else stream
    cfg, dev, buf = ctx["cfg"], ctx["dev"], ctx["buf"]
    gather, fp8 = ctx["dispatch"] == "gather", ctx["dispatch"] in ("fp8", "fp8gemm")
    fp8gemm = ctx["dispatch"] == "fp8gemm"
    calls = {
        "route": lambda: B.moe_route(cfg, dev["x"], dev["w_router"], dev["bias"], buf["logits"],
                                     buf["topk_idx"], buf["topk_w"], ctx["ws_route"], stream),
        "permute": lambda: B.moe_permute(
            cfg, None if (gather or fp8) else dev["x"], buf["topk_idx"], buf["expert_offsets"],
            buf["rank_offsets"], buf["slot_of"], buf["src_of"],
            None if (gather or fp8) else buf["x_perm"], ctx["ws_permute"], stream),
    }
    if fp8:
        calls["fp8_quantize"] = lambda: B.moe_quantize_fp8(cfg, dev["x"], buf["codes"],
                                                           buf["scale_zero"], stream)
    if fp8 and not fp8gemm:
        calls["fp8_dequantize"] = lambda: B.moe_dequantize_fp8(
            cfg, buf["codes"], buf["src_of"], buf["scale_zero"], buf["x_perm"], stream)
    if ctx["ffn"] == "packed":
        pgu, pd = ctx["packed"]
        if fp8gemm:
            calls["ffn_gate_up"] = lambda: B.moe_ffn_gate_up_fp8_gather(
                cfg, buf["codes"], buf["scale_zero"], buf["src_of"], buf["expert_offsets"],
                ctx["fp8_image"], buf["h"], stream)
        elif ctx["backward"]:  # training forward: also keep the pre-activations a and u
            calls["ffn_gate_up"] = lambda: B.moe_ffn_gate_up_packed_train(
                cfg, buf["x_perm"], None, buf["expert_offsets"], pgu, buf["h"], buf["a"],
                buf["u"], stream)
        elif gather:
            calls["ffn_gate_up"] = lambda: B.moe_ffn_gate_up_packed_gather(
                cfg, dev["x"], buf["src_of"], buf["expert_offsets"], pgu, buf["h"], stream)
        else:
            calls["ffn_gate_up"] = lambda: B.moe_ffn_gate_up_packed(
                cfg, buf["x_perm"], buf["expert_offsets"], pgu, buf["h"], stream)
        calls["ffn_down"] = lambda: B.moe_ffn_down_packed(cfg, buf["h"], buf["expert_offsets"],
                                                          pd, buf["y_perm"], stream)
    else:
        calls["ffn_gate_up"] = lambda: B.moe_ffn_gate_up(
            cfg, buf["x_perm"], buf["expert_offsets"], dev["w_gate"], dev["w_up"], buf["h"],
            stream)
        calls["ffn_down"] = lambda: B.moe_ffn_down(cfg, buf["h"], buf["expert_offsets"],
                                                   dev["w_down"], buf["y_perm"], stream)
    calls["combine"] = lambda: B.moe_combine(cfg, buf["y_perm"], buf["slot_of"], buf["topk_w"],
                                             buf["out"], stream)
    return calls


# ----------------------------------------------------------------------------- accounting
def algorithmic(shape, counts, gather=False, fp8gemm=False):
    """Algorithmic HBM bytes and flops of one launch of every phase.  With the
    gather fused into the first GEMM, the dispatch writes indices only and the
    first GEMM reads the token rows (and src_of) instead of x_perm."""
    s = 2 if shape.dtype == "bf16" else 4
    T, d, E, k, f = shape.T, shape.d, shape.E, shape.k, shape.f
    A = T * k
    e_nz = int((counts > 0).sum())
    return {
        "route": dict(bytes=T * d * s + E * d * s + T * E * 4 + 8 * A, flops=2 * T * d * E),
        "permute": dict(bytes=(0 if gather else T * d * s + A * d * s) + 4 * A + 8 * A + 8 * (E + 1),
                        flops=0),
        "ffn_gate_up": dict(bytes=2 * e_nz * f * d * s + A * d * s + A * f * s + (4 * A if gather else 0),
                            flops=2 * A * d * 2 * f),
        "ffn_down": dict(bytes=e_nz * d * f * s + A * f * s + A * d * s, flops=2 * A * f * d),
        "combine": dict(bytes=A * d * s + T * d * s + 8 * A, flops=2 * A * d),
        # logits read once (plus the bias), per-token partials out and back, offsets in
        "route_stats": dict(bytes=T * E * 4 + E * 4 + 16 * T + 8 * (E + 1), flops=0),
        # the row in, one byte per element and (scale, zero) out
        "fp8_quantize": dict(bytes=T * d * s + T * d + 8 * T, flops=0),
        # codes of each row's token (and its scale) in, src_of in, the bf16 row out
        "fp8_dequantize": dict(bytes=A * d + 8 * A + 4 * A + A * d * s, flops=0),
        # d_out and y_perm in, dy_perm out, indices and gates
        "combine_bwd": dict(bytes=T * d * s + 2 * A * d * s + 12 * A, flops=4 * A * d),
        # weights read by the recompute (Wg, Wu), dh (Wd) and dx (Wg, Wu); the three
        # weight gradients written; x_perm and dy read twice each; a, u, h, dh written,
        # then a, u, dh read and h, da, du written by the SwiGLU step, h, da, du read
        # twice each by the products.  16 A d f flops: recompute 4, dh 2, dWd 2, dx 4,
        # dWg + dWu 4.
        "ffn_bwd": dict(bytes=5 * e_nz * f * d * s + 3 * E * f * d * s + 5 * A * d * s
                        + 13 * A * f * s + 8 * (E + 1), flops=16 * A * d * f),
        # logits, bias, indices and gate gradients in; dz out (fp32 + bf16); x, Wr in;
        # dz Wr and dz^T x out
        "route_bwd": dict(bytes=T * E * 4 * 2 + T * E * 2 + 8 * A + T * d * s * 2
                          + 2 * E * d * s, flops=4 * T * E * d),
        "unpermute_bwd": dict(bytes=A * d * s + 2 * T * d * s + 4 * A, flops=A * d),
    } if not fp8gemm else {
        **algorithmic(shape, counts, gather=True),
        # E4M3 weight codes of every expert with rows (read once) and their per-row scale and
        # code sum, the token codes gathered through src_of (one row each, plus src_of and the
        # token's scale and centre), h out
        "ffn_gate_up": dict(bytes=2 * e_nz * f * d + 2 * e_nz * f * 8 + A * d + 12 * A
                            + A * f * s, flops=2 * A * d * 2 * f, peak="fp8"),
    }


def roofline_of(work, ms, dtype="bf16"):
    """Achieved rate against the roofline the kernel's arithmetic intensity
    selects (HBM below the ridge, the matrix-core or vector peak above)."""
    sec = ms * 1e-3
    peak_fl = PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_FP32_TFLOPS
    if work.get("peak") == "fp8":
        peak_fl = PEAK_FP8_TFLOPS
    ai = work["flops"] / work["bytes"] if work["bytes"] else float("inf")
    ridge = peak_fl * 1e12 / (PEAK_HBM_GBS * 1e9)
    gbs = work["bytes"] / sec / 1e9
    tfl = work["flops"] / sec / 1e12
    if ai < ridge:
        return dict(bound="hbm", achieved=gbs, peak=PEAK_HBM_GBS, unit="GB/s", frac=gbs / PEAK_HBM_GBS,
                    tflops=tfl, mfma_frac=tfl / peak_fl, ai=ai)
    return dict(bound="mfma" if (dtype == "bf16" or work.get("peak") == "fp8") else "alu",
                achieved=tfl, peak=peak_fl,
                unit="TFLOP/s", frac=tfl / peak_fl, gbs=gbs, hbm_frac=gbs / PEAK_HBM_GBS, ai=ai)


def measured_traffic(ffn, workload, dispatch):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None if there is none, it is for another workload or dispatch
    mode, or the kernel source changed since."""
    traffic_file, kernel_srcs, _ = FFN_KERNELS[ffn]
    try:
        with open(traffic_file) as fh:
            t = json.load(fh)
        h = kernel_sources_sha256(kernel_srcs)
    except (OSError, ValueError):
        return None
    if (t.get("kernel_src_sha256") != h or t.get("workload") != workload or
            t.get("dispatch", "copy") != dispatch):
        return None
    return t.get("bytes_per_launch")


# ----------------------------------------------------------------------------- oracle leg
def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(shape, inp, n_tok):
    """The CPU oracle as it stands, on the first n_tok tokens (whole layer)."""
    import oracle
    n_tok = min(n_tok, shape.T)
    t0 = time.perf_counter()
    oracle.layer(inp["x"][:n_tok], inp["w_router"], inp["bias"], inp["w_gate"], inp["w_up"],
                 inp["w_down"], k=shape.k, n_group=shape.n_group, topk_group=shape.topk_group,
                 presel=shape.presel, renorm=shape.renorm, ep_ranks=shape.ep_ranks)
    dt = time.perf_counter() - t0
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": _oracle_threads(), "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"first {n_tok} of {shape.T} tokens, whole layer (route, permute, FFN, "
                      f"combine) in float64 NumPy; {dt:.1f} s"}


def routing_flips(shape, inp, idx_gpu):
    """Tokens whose chosen set differs from the oracle's float64 routing of
    the same inputs; every one must sit at a selection margin below 1e-4."""
    import numpy as np
    import oracle
    z64 = oracle.router_logits(inp["x"], inp["w_router"])
    s64 = z64 + (0.0 if inp["bias"] is None else inp["bias"].astype(np.float64)[None, :])
    o_idx, _, _ = oracle.route(z64.astype(np.float32), inp["bias"], k=shape.k,
                               n_group=shape.n_group, topk_group=shape.topk_group,
                               presel=shape.presel, renorm=shape.renorm)
    flip = np.any(np.sort(idx_gpu, 1) != np.sort(o_idx, 1), axis=1)
    margin = oracle.margins(s64, shape.k, shape.n_group, shape.topk_group)
    near = margin < FLIP_MARGIN
    return {"tokens": int(shape.T), "flips": int(flip.sum()),
            "flips_outside_margin": int((flip & ~near).sum()),
            "near_ties": int(near.sum()), "margin": FLIP_MARGIN}


# ----------------------------------------------------------------------------- timing
def copy_bandwidth(nbytes=1 << 31, reps=10):
    """Plain device-to-device copy, read + write bytes per second (GB/s)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(reps):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)


def time_steps(ctx, calls, phases_run, steps, warmup, flush_pass=True):
    """W warm-ups, K timed steps (one event pair around the dominant kernel in
    each), then the same steps untimed with an event after every phase for the
    breakdown, and optionally once more with the MALL evicted before each step."""
    import numpy as np
    import torch
    stream = torch.cuda.current_stream()

    def step(ev=None, dom_ev=None):
        if ev is not None:
            ev[0].record(stream)
        for i, p in enumerate(phases_run):
            if dom_ev is not None and p == DOMINANT:
                dom_ev[0].record(stream)
            calls[p]()
            if dom_ev is not None and p == DOMINANT:
                dom_ev[1].record(stream)
            if ev is not None:
                ev[i + 1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    dom_events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        step(dom_ev=dom_events[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dom_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in dom_events]))

    def breakdown(flush):
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda") if flush else None
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases_run) + 1)]
                  for _ in range(steps)]
        for s in range(steps):
            if flush:  # 1 GiB written: nothing of the previous step stays in the 256 MB MALL
                scratch.fill_(s & 0xFF)
            step(ev=events[s])
        torch.cuda.synchronize()
        return {p: float(np.mean([events[s][i].elapsed_time(events[s][i + 1])
                                  for s in range(steps)])) for i, p in enumerate(phases_run)}, \
            float(np.mean([events[s][0].elapsed_time(events[s][-1]) for s in range(steps)]))

    phase_ms, _ = breakdown(False)
    phase_ms[DOMINANT] = dom_ms  # the dominant kernel as timed inside the timed region
    flushed = None
    if flush_pass:
        fl_ms, fl_step = breakdown(True)
        flushed = {"ms_per_step": round(fl_step, 5), **{p: round(v, 5) for p, v in fl_ms.items()}}
    return elapsed, phase_ms, flushed


def run_forward(shape, a, inp, copy_gbs=None, headline=True):
    """Times one workload's forward; returns the record of its line."""
    import numpy as np
    import torch
    from top_routing_expert_amd import binding as B

    ctx = prepare(shape, inp, a.ffn, a.dispatch, a.backward)
    calls = forward_calls(ctx)
    phases_run = tuple(calls)
    cfg, dev, buf = ctx["cfg"], ctx["dev"], ctx["buf"]
    T, E, k, d, f, R = shape.T, shape.E, shape.k, shape.d, shape.f, shape.ep_ranks
    A = T * k
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    stream = torch.cuda.current_stream()
    if a.diagnostics:
        buf["hist"] = torch.empty(E, dtype=torch.int32, device="cuda")
        buf["rload"] = torch.empty(R, dtype=torch.int32, device="cuda")
        buf["stats"] = torch.empty(4, dtype=torch.float32, device="cuda")
        ws_s = B.workspace(cfg, "route_stats")
        calls["route_stats"] = lambda: B.moe_route_stats(
            cfg, buf["logits"], dev["bias"], buf["expert_offsets"], buf["rank_offsets"],
            buf["hist"], buf["rload"], buf["stats"], ws_s, stream)
        phases_run = phases_run[:2] + ("route_stats",) + phases_run[2:]
    if a.backward:
        buf["a"] = torch.empty((A, f), dtype=dt, device="cuda")
        buf["u"] = torch.empty((A, f), dtype=dt, device="cuda")
        from top_routing_expert_amd import inputs as I
        grad = dict(
            dout=B.to_device(I.make_grad_out(shape, seed_of(shape))),
            dy=torch.empty((A, d), dtype=dt, device="cuda"),
            dw=torch.empty((T, k), dtype=torch.float32, device="cuda"),
            dxp=torch.empty((A, d), dtype=dt, device="cuda"),
            dwg=torch.empty((E, f, d), dtype=dt, device="cuda"),
            dwu=torch.empty((E, f, d), dtype=dt, device="cuda"),
            dwd=torch.empty((E, d, f), dtype=dt, device="cuda"),
            dz=torch.empty((T, E), dtype=torch.float32, device="cuda"),
            dxr=torch.empty((T, d), dtype=dt, device="cuda"),
            dwr=torch.empty((E, d), dtype=dt, device="cuda"),
            db=torch.empty(E, dtype=torch.float32, device="cuda") if dev["bias"] is not None else None,
            dx=torch.empty((T, d), dtype=dt, device="cuda"),
        )
        ws_fb, ws_rb = B.workspace(cfg, "ffn_backward"), B.workspace(cfg, "route_backward")
        images = (None, None)
        if ctx["ffn"] == "packed":  # the transposed images for dh and dx, packed once
            images = B.pack_weights_backward(cfg, dev["w_gate"], dev["w_up"], dev["w_down"],
                                             stream=stream)
            torch.cuda.synchronize()
        calls["combine_bwd"] = lambda: B.moe_combine_backward(
            cfg, grad["dout"], buf["y_perm"], buf["slot_of"], buf["topk_w"], grad["dy"],
            grad["dw"], stream)
        calls["ffn_bwd"] = lambda: B.moe_ffn_backward(
            cfg, buf["x_perm"], buf["expert_offsets"], dev["w_gate"], dev["w_up"], dev["w_down"],
            grad["dy"], grad["dxp"], grad["dwg"], grad["dwu"], grad["dwd"], ws_fb, stream,
            a=buf.get("a"), u=buf.get("u"), packed_dh=images[0], packed_dx=images[1])
        calls["route_bwd"] = lambda: B.moe_route_backward(
            cfg, dev["x"], dev["w_router"], buf["logits"], dev["bias"], buf["topk_idx"],
            grad["dw"], grad["dz"], grad["dxr"], grad["dwr"], grad["db"], ws_rb, stream)
        calls["unpermute_bwd"] = lambda: B.moe_unpermute_backward(
            cfg, grad["dxp"], buf["slot_of"], grad["dxr"], grad["dx"], stream)
        phases_run = phases_run + ("combine_bwd", "ffn_bwd", "route_bwd", "unpermute_bwd")

    log(f"{shape.name}: warmup {a.warmup}, timing {a.steps} steps")
    elapsed, phase_ms, flushed = time_steps(ctx, calls, phases_run, a.steps, a.warmup,
                                            flush_pass=not a.no_flush_pass)
    counts = np.diff(B.to_host_bits(buf["expert_offsets"]).astype(np.int64))
    idx_gpu = B.to_host_bits(buf["topk_idx"])
    gather = ctx["dispatch"] == "gather"
    work = algorithmic(shape, counts, gather, fp8gemm=ctx["dispatch"] == "fp8gemm")
    if a.backward and ctx["ffn"] == "packed":  # the saved pre-activations, written by the forward
        work["ffn_gate_up"]["bytes"] += 2 * A * f * (2 if shape.dtype == "bf16" else 4)
        # and read by the backward instead of the recompute (no weight re-read, 4 A d f fewer flops)
        work["ffn_bwd"]["bytes"] -= 2 * int((counts > 0).sum()) * f * d * 2
        work["ffn_bwd"]["flops"] -= 4 * A * d * f
    phases = {p: dict(ms=phase_ms[p], **roofline_of(work[p], phase_ms[p], shape.dtype))
              for p in phases_run}
    dom = phases[DOMINANT]
    traffic = measured_traffic(ctx["ffn"], shape.name, ctx["dispatch"])
    roofline = {"bound": dom["bound"], "achieved": round(dom["achieved"], 3),
                "peak": dom["peak"], "unit": dom["unit"], "frac": round(dom["frac"], 4),
                "traffic": traffic,
                "kernel": ("gate_up_fp8_kernel (moe_ffn_gate_up_fp8_gather)"
                           if ctx["dispatch"] == "fp8gemm" else FFN_KERNELS[ctx["ffn"]][2].replace(
                    ")", "_gather)" if gather else ("_train)" if a.backward and ctx["ffn"] == "packed" else ")"))),
                "algorithmic_bytes": work[DOMINANT]["bytes"],
                "algorithmic_flops": work[DOMINANT]["flops"],
                "avg_launch_ms": round(dom["ms"], 5)}
    if copy_gbs and dom["unit"] == "GB/s":
        roofline["measured_copy_gbs"] = round(copy_gbs, 1)
        roofline["frac_of_measured_copy"] = round(dom["achieved"] / copy_gbs, 4)
    rec = {
        "value": T * a.steps / elapsed,
        "ms_per_step": elapsed * 1e3 / a.steps,
        "dtype": shape.dtype,
        "config": {"workload": shape.name, "T": T, "d": d, "E": E, "k": k, "f": f,
                   "n_group": shape.n_group, "topk_group": shape.topk_group,
                   "presel": shape.presel, "renorm": shape.renorm, "ep_ranks": R,
                   "ffn_weights": ctx["ffn"], "dispatch": ctx["dispatch"],
                   "backward": a.backward, "parallelism": "single GPU"},
        "roofline": roofline,
        "phases": {p: {kk: (round(v, 5) if isinstance(v, float) else v) for kk, v in ph.items()}
                   for p, ph in phases.items()},
        "phases_mall_flushed": flushed,
        "expert_rows": {"min": int(counts.min()), "max": int(counts.max()),
                        "empty": int((counts == 0).sum())},
    }
    # phase fractions against their own rooflines, for the summary
    if copy_gbs:
        for p in phases_run:
            if rec["phases"][p]["unit"] == "GB/s":
                rec["phases"][p]["frac_of_measured_copy"] = round(
                    rec["phases"][p]["achieved"] / copy_gbs, 4)
    del ctx, calls, dev, buf
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec, idx_gpu


def time_variants(shape, a, inp, copy_gbs):
    """The rows built beside the timed path, timed on the same workload: the FP8
    first GEMM (per-token FP8 codes x E4M3 expert weights; a different model,
    so never the line's value) and the layer in expert waves (bit for bit the
    serial layer).  A failure is recorded, not raised: the line stays."""
    import argparse as _ap
    import torch
    from top_routing_expert_amd import binding as B

    out = {}
    if shape.dtype != "bf16":
        return out
    try:
        va = _ap.Namespace(**vars(a))
        va.dispatch, va.no_flush_pass = "fp8gemm", True
        va.steps, va.warmup = min(a.steps, 10), min(a.warmup, 3)
        rec, _ = run_forward(shape, va, inp, copy_gbs, headline=False)
        ph = rec["phases"]["ffn_gate_up"]
        out["fp8_first_gemm"] = dict(
            value=rec["value"], unit="tokens/s", ms_per_step=rec["ms_per_step"],
            ffn_gate_up_ms=ph["ms"], ffn_gate_up_tflops=ph.get("tflops", ph.get("achieved")),
            ffn_gate_up_frac_of_fp8_peak=ph.get("mfma_frac", ph.get("frac")),
            roofline=rec["roofline"], steps=va.steps,
            note="per-token E4M3 codes x per-output-channel E4M3 gate/up weights; bf16 down")
    except Exception as e:  # pragma: no cover
        out["fp8_first_gemm"] = {"error": repr(e)}
    try:
        log(f"{shape.name}: expert waves")
        ctx = prepare(shape, inp)
        cfg, dev, buf = ctx["cfg"], ctx["dev"], ctx["buf"]
        pgu, pd = ctx["packed"]
        ws = B.workspace(cfg, "layer")
        bufs = {n: buf[n] for n in ("logits", "topk_idx", "topk_w", "expert_offsets",
                                    "rank_offsets", "slot_of", "src_of", "h", "y_perm")}
        aux = torch.cuda.Stream()  # default priority
        runs = {"serial": lambda: B.moe_layer_fwd_packed(cfg, dev["x"], dev["w_router"],
                                                         dev["bias"], pgu, pd, buf["out"], bufs,
                                                         ws)}
        for W in (2, 4):
            if shape.E % W == 0:
                runs[f"{W}_waves"] = (lambda W=W: B.moe_layer_fwd_packed_waved(
                    cfg, dev["x"], dev["w_router"], dev["bias"], pgu, pd, buf["out"], bufs, ws,
                    n_waves=W, aux_stream=aux))
        for f in runs.values():
            f()
            f()
        torch.cuda.synchronize()
        ms = {k: [] for k in runs}
        for _ in range(5):
            for k, f in runs.items():
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                ev[0].record()
                for _ in range(4):
                    f()
                ev[1].record()
                torch.cuda.synchronize()
                ms[k].append(ev[0].elapsed_time(ev[1]) / 4)
        med = {k: round(sorted(v)[len(v) // 2], 5) for k, v in ms.items()}
        out["expert_waves"] = dict(ms_per_layer=med, unit="ms",
                                   note="moe_layer_fwd_packed vs moe_layer_fwd_packed_waved "
                                        "(two streams), median of 5 x 4 calls")
        del ctx
    except Exception as e:  # pragma: no cover
        out["expert_waves"] = {"error": repr(e)}
    return out


def main(argv=None):
    a = parse(argv)
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {a.gpus} requested): this path has no "
              "multi-GPU mode; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    from top_routing_expert_amd import inputs as I

    if a.copy_calibration:
        copy_calibration()
        return
    if a.backward and a.shape.dtype != "bf16":
        print("--backward needs a bf16 workload", file=sys.stderr)
        sys.exit(2)
    log("copy bandwidth")
    copy_gbs = copy_bandwidth()
    shape = a.shape
    log(f"workload {shape.name}: generating inputs")
    inp = I.make_inputs(shape, seed=seed_of(shape))
    rec, idx_gpu = run_forward(shape, a, inp, copy_gbs)
    variants = time_variants(shape, a, inp, copy_gbs) if a.variants == "all" else None
    cpu = flips = None
    if a.cpu_tokens > 0:
        log(f"oracle leg: CPU baseline on {a.cpu_tokens} tokens, routing flips over all tokens")
        cpu = cpu_baseline(shape, inp, a.cpu_tokens)
        flips = routing_flips(shape, inp, idx_gpu)
    del inp
    others = {}
    for o in a.others:
        if o == shape:
            continue
        log(f"workload {o.name}: generating inputs")
        oin = I.make_inputs(o, seed=seed_of(o))
        orec, oidx = run_forward(o, a, oin, copy_gbs, headline=False)
        if a.cpu_tokens > 0:
            orec["flips"] = routing_flips(o, oin, oidx)
        del oin
        others[o.name] = {kk: orec[kk] for kk in ("value", "ms_per_step", "dtype", "roofline",
                                                   "phases", "phases_mall_flushed", "expert_rows")}
        others[o.name]["unit"] = "tokens/s"
        if "flips" in orec:
            others[o.name]["flips"] = orec["flips"]
    res = {
        "metric": ("MoE-layer fwd+bwd tokens/s @1 GPU (training step)" if a.backward else
                   "MoE-layer fwd tokens/s @1 GPU; % bf16 MFMA peak (FFN), % HBM BW (route/permute)"),
        "value": rec["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": rec["dtype"],
        "data": "synthetic (seeded Gaussian inputs and random-init expert weights)",
        "config": rec["config"],
        "roofline": rec["roofline"],
        "cpu_baseline": cpu,
        "flips": flips,
        "phases": rec["phases"],
        "phases_mall_flushed": rec["phases_mall_flushed"],
        "expert_rows": rec["expert_rows"],
        "measured_copy_gbs": round(copy_gbs, 1),
        "workloads": others,
    }
    if variants is not None:
        res["variants"] = variants
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
