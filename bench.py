#!/usr/bin/env python3
"""MoE-layer forward throughput on one MI355X.

One step = one pass of the whole path over one batch of synthetic tokens:
moe_route -> moe_permute -> moe_ffn_gate_up -> moe_ffn_down -> moe_combine,
each a C-ABI call that enqueues the HIP kernels on the current stream.  With
the packed FFN the dispatch's row gather runs inside the first GEMM by default
(moe_permute writes the indices, moe_ffn_gate_up_packed_gather reads the token
rows through src_of); --dispatch copy materialises x_perm first.
Inputs are resident in HBM before timing starts.  W warm-up steps, then K
timed steps bracketed by device synchronisation; HIP events recorded on the
same stream between the calls give each kernel's average duration inside the
timed region.  Prints ONE JSON line (rank 0).

Default workload: T=1024 tokens, d=4096, E=8 experts, top-2, SwiGLU f=11008,
bf16 (the headline workload of the method's metric).
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
PHASES = ("route", "permute", "ffn_gate_up", "ffn_down", "combine")
DOMINANT = "ffn_gate_up"
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


def parse():
    from top_routing_expert_amd import configs as C
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="2",
                    help="workload index 1..5 or name; default 2 (T1024-d4096-E8-top2-f11008)")
    ap.add_argument("--cpu-tokens", type=int, default=256,
                    help="tokens of the workload the CPU oracle baseline runs (0 = skip)")
    ap.add_argument("--ffn", choices=sorted(FFN_KERNELS), default="packed",
                    help="expert-weight layout of the grouped FFN: packed once at load time "
                         "(moe_pack_weights) or the plain [E,f,d] / [E,d,f] arrays")
    ap.add_argument("--dispatch", choices=("gather", "copy", "fp8"), default="gather",
                    help="packed FFN: gather the token rows inside the first GEMM (the dispatch "
                         "writes indices only), copy them to x_perm first, or send them as "
                         "per-token FP8 (quantize, then decode into x_perm in expert order)")
    ap.add_argument("--diagnostics", action="store_true",
                    help="also time the routing diagnostics (moe_route_stats) after the dispatch; "
                         "reported as its own phase and included in the step")
    ap.add_argument("--backward", action="store_true",
                    help="time forward + backward (combine, grouped FFN, router and dispatch "
                         "backward on the forward's routing) instead of the forward alone")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for counter calibration)")
    a = ap.parse_args()
    if a.config.isdigit():
        a.shape = C.CONFIGS[int(a.config) - 1]
    else:
        a.shape = C.BY_NAME[a.config]
    return a


def algorithmic(shape, counts, gather=False):
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
    }


def roofline_of(work, ms):
    sec = ms * 1e-3
    ai = work["flops"] / work["bytes"] if work["bytes"] else float("inf")
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    gbs = work["bytes"] / sec / 1e9
    tfl = work["flops"] / sec / 1e12
    if ai < ridge:
        return dict(bound="hbm", achieved=gbs, peak=PEAK_HBM_GBS, unit="GB/s", frac=gbs / PEAK_HBM_GBS,
                    tflops=tfl, mfma_frac=tfl / PEAK_BF16_TFLOPS, ai=ai)
    return dict(bound="mfma", achieved=tfl, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                frac=tfl / PEAK_BF16_TFLOPS, gbs=gbs, hbm_frac=gbs / PEAK_HBM_GBS, ai=ai)


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


def cpu_baseline(shape, inp, n_tok):
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    n_tok = min(n_tok, shape.T)
    t0 = time.perf_counter()
    oracle.layer(inp["x"][:n_tok], inp["w_router"], inp["bias"], inp["w_gate"], inp["w_up"],
                 inp["w_down"], k=shape.k, n_group=shape.n_group, topk_group=shape.topk_group,
                 presel=shape.presel, renorm=shape.renorm, ep_ranks=shape.ep_ranks)
    dt = time.perf_counter() - t0
    del np
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {n_tok} of {shape.T} tokens, whole layer (route, permute, FFN, "
                      f"combine) in float64 NumPy; {dt:.1f} s"}


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {a.gpus} requested): this path has no "
              "multi-GPU mode; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from top_routing_expert_amd import binding as B
    from top_routing_expert_amd import inputs as I

    if a.copy_calibration:
        copy_calibration()
        return
    shape = a.shape
    if shape.dtype != "bf16":
        a.ffn = "rowmajor"  # packed images are bf16 only
    if a.ffn != "packed":
        a.dispatch = "copy"  # the gather is a packed-FFN kernel
    if a.backward:
        if shape.dtype != "bf16":
            print("--backward needs a bf16 workload", file=sys.stderr)
            sys.exit(2)
        a.dispatch = "copy"  # the FFN backward reads the dispatched rows
    gather = a.dispatch == "gather"
    fp8 = a.dispatch == "fp8"
    log(f"workload {shape.name}: generating inputs")
    from top_routing_expert_amd import configs as C
    inp = I.make_inputs(shape, seed=C.CONFIGS.index(shape) + 1)
    dev = {k: (None if v is None else B.to_device(v)) for k, v in inp.items()}
    cfg = B.config(shape)
    T, E, k, d, f, R = shape.T, shape.E, shape.k, shape.d, shape.f, shape.ep_ranks
    A = T * k
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    buf = dict(
        logits=torch.empty((T, E), dtype=torch.float32, device="cuda"),
        idx=torch.empty((T, k), dtype=torch.int32, device="cuda"),
        w=torch.empty((T, k), dtype=torch.float32, device="cuda"),
        offs=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
        roffs=torch.empty(R + 1, dtype=torch.int32, device="cuda"),
        slot=torch.empty(A, dtype=torch.int32, device="cuda"),
        src=torch.empty(A, dtype=torch.int32, device="cuda"),
        xp=None if gather else torch.empty((A, d), dtype=dt, device="cuda"),
        codes=torch.empty((T, d), dtype=torch.uint8, device="cuda") if fp8 else None,
        sz=torch.empty((T, 2), dtype=torch.float32, device="cuda") if fp8 else None,
        h=torch.empty((A, f), dtype=dt, device="cuda"),
        y=torch.empty((A, d), dtype=dt, device="cuda"),
        out=torch.empty((T, d), dtype=dt, device="cuda"),
    )
    ws_r, ws_p = B.workspace(cfg, "route"), B.workspace(cfg, "permute")
    stream = torch.cuda.current_stream()
    if a.ffn == "packed":
        # load-time weight layout: packed once, the plain arrays are then dropped
        log("packing expert weights")
        pgu, pd = B.pack_weights(cfg, dev["w_gate"], dev["w_up"], dev["w_down"], stream=stream)
        torch.cuda.synchronize()
        if not a.backward:  # the backward reads the weights in their own layout
            dev["w_gate"] = dev["w_up"] = dev["w_down"] = None
        if a.backward:  # training forward: also keep the pre-activations a and u
            buf["a"] = torch.empty((A, f), dtype=dt, device="cuda")
            buf["u"] = torch.empty((A, f), dtype=dt, device="cuda")
            gate_up = lambda: B.moe_ffn_gate_up_packed_train(cfg, buf["xp"], None, buf["offs"], pgu,
                                                              buf["h"], buf["a"], buf["u"], stream)
        elif a.dispatch == "gather":
            gate_up = lambda: B.moe_ffn_gate_up_packed_gather(cfg, dev["x"], buf["src"],
                                                               buf["offs"], pgu, buf["h"], stream)
        else:
            gate_up = lambda: B.moe_ffn_gate_up_packed(cfg, buf["xp"], buf["offs"], pgu,
                                                        buf["h"], stream)
        ffn_calls = {
            "ffn_gate_up": gate_up,
            "ffn_down": lambda: B.moe_ffn_down_packed(cfg, buf["h"], buf["offs"], pd, buf["y"],
                                                      stream),
        }
    else:
        ffn_calls = {
            "ffn_gate_up": lambda: B.moe_ffn_gate_up(cfg, buf["xp"], buf["offs"], dev["w_gate"],
                                                     dev["w_up"], buf["h"], stream),
            "ffn_down": lambda: B.moe_ffn_down(cfg, buf["h"], buf["offs"], dev["w_down"],
                                               buf["y"], stream),
        }

    calls = {
        "route": lambda: B.moe_route(cfg, dev["x"], dev["w_router"], dev["bias"], buf["logits"],
                                     buf["idx"], buf["w"], ws_r, stream),
        "permute": lambda: B.moe_permute(cfg, None if (gather or fp8) else dev["x"], buf["idx"],
                                         buf["offs"], buf["roffs"], buf["slot"], buf["src"],
                                         None if (gather or fp8) else buf["xp"], ws_p, stream),
        **ffn_calls,
        "combine": lambda: B.moe_combine(cfg, buf["y"], buf["slot"], buf["w"], buf["out"], stream),
    }
    phases_run = PHASES
    if fp8:
        calls["fp8_quantize"] = lambda: B.moe_quantize_fp8(cfg, dev["x"], buf["codes"], buf["sz"],
                                                           stream)
        calls["fp8_dequantize"] = lambda: B.moe_dequantize_fp8(cfg, buf["codes"], buf["src"],
                                                               buf["sz"], buf["xp"], stream)
        phases_run = PHASES[:2] + ("fp8_quantize", "fp8_dequantize") + PHASES[2:]
    if a.diagnostics:
        buf["hist"] = torch.empty(E, dtype=torch.int32, device="cuda")
        buf["rload"] = torch.empty(R, dtype=torch.int32, device="cuda")
        buf["stats"] = torch.empty(4, dtype=torch.float32, device="cuda")
        ws_s = B.workspace(cfg, "route_stats")
        calls["route_stats"] = lambda: B.moe_route_stats(cfg, buf["logits"], dev["bias"], buf["offs"],
                                                         buf["roffs"], buf["hist"], buf["rload"],
                                                         buf["stats"], ws_s, stream)
        phases_run = phases_run[:2] + ("route_stats",) + phases_run[2:]

    if a.backward:
        grad = dict(
            dout=B.to_device(I.make_grad_out(shape, C.CONFIGS.index(shape) + 1)),
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
        if a.ffn == "packed":  # the transposed images for dh and dx, packed once like pgu / pd
            images = B.pack_weights_backward(cfg, dev["w_gate"], dev["w_up"], dev["w_down"],
                                             stream=stream)
            torch.cuda.synchronize()
        calls["combine_bwd"] = lambda: B.moe_combine_backward(
            cfg, grad["dout"], buf["y"], buf["slot"], buf["w"], grad["dy"], grad["dw"], stream)
        calls["ffn_bwd"] = lambda: B.moe_ffn_backward(
            cfg, buf["xp"], buf["offs"], dev["w_gate"], dev["w_up"], dev["w_down"], grad["dy"],
            grad["dxp"], grad["dwg"], grad["dwu"], grad["dwd"], ws_fb, stream, a=buf.get("a"),
            u=buf.get("u"), packed_dh=images[0], packed_dx=images[1])
        calls["route_bwd"] = lambda: B.moe_route_backward(
            cfg, dev["x"], dev["w_router"], buf["logits"], dev["bias"], buf["idx"], grad["dw"],
            grad["dz"], grad["dxr"], grad["dwr"], grad["db"], ws_rb, stream)
        calls["unpermute_bwd"] = lambda: B.moe_unpermute_backward(
            cfg, grad["dxp"], buf["slot"], grad["dxr"], grad["dx"], stream)
        phases_run = phases_run + ("combine_bwd", "ffn_bwd", "route_bwd", "unpermute_bwd")

    def step(ev=None, dom_ev=None):
        """One pass of the path.  ev: an event after every phase (the phase
        breakdown); dom_ev: one pair around the dominant kernel only (the
        timed steps: six markers per step cost ~3 % of the T1024 step)."""
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

    log(f"warmup {a.warmup}")
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    counts = np.diff(B.to_host_bits(buf["offs"]).astype(np.int64))
    dom_events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(a.steps)]
    log(f"timing {a.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(a.steps):
        step(dom_ev=dom_events[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dom_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in dom_events]))
    # phase breakdown: the same steps again, untimed, with an event after every phase
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases_run) + 1)]
              for _ in range(a.steps)]
    for s in range(a.steps):
        step(ev=events[s])
    torch.cuda.synchronize()
    phase_ms = {p: float(np.mean([events[s][i].elapsed_time(events[s][i + 1])
                                  for s in range(a.steps)])) for i, p in enumerate(phases_run)}
    phase_ms[DOMINANT] = dom_ms  # the dominant kernel as timed inside the timed region
    ms_per_step = elapsed * 1e3 / a.steps
    work = algorithmic(shape, counts, gather)
    if a.backward and a.ffn == "packed":  # the saved pre-activations, written by the forward
        work["ffn_gate_up"]["bytes"] += 2 * A * f * (2 if shape.dtype == "bf16" else 4)
        # and read by the backward instead of the recompute (no weight re-read, 4 A d f fewer flops)
        work["ffn_bwd"]["bytes"] -= 2 * int((counts > 0).sum()) * f * d * 2
        work["ffn_bwd"]["flops"] -= 4 * A * d * f
    phases = {p: dict(ms=phase_ms[p], **roofline_of(work[p], phase_ms[p])) for p in phases_run}
    dom = phases[DOMINANT]
    traffic = measured_traffic(a.ffn, shape.name, a.dispatch)
    roofline = {"bound": dom["bound"], "achieved": round(dom["achieved"], 3),
                "peak": dom["peak"], "unit": dom["unit"], "frac": round(dom["frac"], 4),
                "traffic": traffic,
                "kernel": FFN_KERNELS[a.ffn][2].replace(
                    ")", "_gather)" if gather else ("_train)" if a.backward and a.ffn == "packed" else ")")),
                "algorithmic_bytes": work[DOMINANT]["bytes"],
                "algorithmic_flops": work[DOMINANT]["flops"],
                "avg_launch_ms": round(dom["ms"], 5)}
    cpu = None
    if a.cpu_tokens > 0:
        log(f"cpu baseline: oracle on {a.cpu_tokens} tokens")
        cpu = cpu_baseline(shape, inp, a.cpu_tokens)
    res = {
        "metric": ("MoE-layer fwd+bwd tokens/s @1 GPU (training step)" if a.backward else
                   "MoE-layer fwd tokens/s @1 GPU; % bf16 MFMA peak (FFN), % HBM BW (route/permute)"),
        "value": T * a.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.dtype,
        "data": "synthetic (seeded Gaussian inputs and random-init expert weights)",
        "config": {"workload": shape.name, "T": T, "d": d, "E": E, "k": k, "f": f,
                   "n_group": shape.n_group, "topk_group": shape.topk_group,
                   "presel": shape.presel, "renorm": shape.renorm, "ep_ranks": R,
                   "ffn_weights": a.ffn, "dispatch": a.dispatch, "backward": a.backward,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "phases": {p: {kk: (round(v, 5) if isinstance(v, float) else v) for kk, v in ph.items()}
                   for p, ph in phases.items()},
        "expert_rows": {"min": int(counts.min()), "max": int(counts.max()),
                        "empty": int((counts == 0).sum())},
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
