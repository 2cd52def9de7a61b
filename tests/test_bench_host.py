"""bench.py's host logic, on the CPU: the default line and its workloads, the
one-GPU refusal, the algorithmic bytes and flops the roofline divides by,
the choice of roofline, and the rule that a committed counter summary is
used only for its own workload, dispatch and kernel sources."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from top_routing_expert_amd import configs as C  # noqa: E402

E256 = "T8192-d7168-E256-g8x4-top8-f2048"


def test_default_line_is_the_largest_workload_with_the_others_and_variants():
    a = bench.parse([])
    assert a.shape.name == E256 and a.gpus == 1
    assert [s.name for s in a.others] == [c.name for c in C.CONFIGS[:4]]
    assert a.variants == "all" and a.dispatch == "gather" and a.ffn == "packed"
    one = bench.parse(["--config", "2"])
    assert one.others == [] and one.variants == "none"
    fp8 = bench.parse(["--dispatch", "fp8gemm"])
    assert fp8.others == [] and fp8.variants == "none"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_gate_up_bytes_and_flops_of_the_largest_workload():
    """Weights of the 256 experts with rows (2 f d bf16 each), the 65 536
    gathered token rows, their src_of entries and h: 16 240 607 232 bytes,
    and 2 A d 2f flops."""
    shape = C.BY_NAME[E256]
    counts = np.full(shape.E, shape.T * shape.k // shape.E)
    w = bench.algorithmic(shape, counts, gather=True)["ffn_gate_up"]
    A, d, f = shape.T * shape.k, shape.d, shape.f
    assert w["bytes"] == 2 * 256 * f * d * 2 + A * d * 2 + 4 * A + A * f * 2 == 16240607232
    assert w["flops"] == 2 * A * d * 2 * f
    # without the gather the dispatch writes x_perm and GEMM1 reads it (no src_of)
    wc = bench.algorithmic(shape, counts, gather=False)
    assert wc["ffn_gate_up"]["bytes"] == w["bytes"] - 4 * A
    assert wc["permute"]["bytes"] > bench.algorithmic(shape, counts, gather=True)["permute"]["bytes"]
    # experts without rows stream no weights
    counts[:16] = 0
    assert (bench.algorithmic(shape, counts, gather=True)["ffn_gate_up"]["bytes"]
            == w["bytes"] - 16 * 2 * f * d * 2)
    # the FP8 first GEMM reads one byte per weight and token element
    w8 = bench.algorithmic(shape, np.ones(shape.E), fp8gemm=True)["ffn_gate_up"]
    assert w8["peak"] == "fp8" and w8["flops"] == w["flops"]
    assert w8["bytes"] == 2 * 256 * f * d + 2 * 256 * f * 8 + A * d + 12 * A + A * f * 2


def test_roofline_follows_arithmetic_intensity():
    ms = 1.0
    hbm = bench.roofline_of(dict(bytes=8e9, flops=1e12), ms)  # 125 flop/B < ridge 312.5
    assert hbm["bound"] == "hbm" and hbm["unit"] == "GB/s"
    assert abs(hbm["achieved"] - 8000.0) < 1e-6 and abs(hbm["frac"] - 1.0) < 1e-9
    mf = bench.roofline_of(dict(bytes=1e9, flops=2.5e12), ms)  # 2500 flop/B
    assert mf["bound"] == "mfma" and mf["unit"] == "TFLOP/s" and abs(mf["frac"] - 1.0) < 1e-9
    f8 = bench.roofline_of(dict(bytes=1e9, flops=1e12, peak="fp8"), ms)  # 1000 > fp8 ridge 625
    assert f8["bound"] == "mfma" and f8["peak"] == bench.PEAK_FP8_TFLOPS
    f8h = bench.roofline_of(dict(bytes=1e9, flops=5e11, peak="fp8"), ms)  # 500 < 625
    assert f8h["bound"] == "hbm" and abs(f8h["mfma_frac"] - 0.1) < 1e-9
    f32 = bench.roofline_of(dict(bytes=1e6, flops=1e12), ms, dtype="f32")
    assert f32["bound"] == "alu" and f32["peak"] == bench.PEAK_FP32_TFLOPS


def test_committed_traffic_is_used_only_for_its_workload_dispatch_and_sources(tmp_path,
                                                                              monkeypatch):
    path, srcs, name = bench.FFN_KERNELS["packed"]
    with open(path) as fh:
        t = json.load(fh)
    assert t["workload"] == E256 and t["dispatch"] == "gather"
    # counter bytes = FETCH_SIZE x its copy scale + WRITE_SIZE x its copy scale
    got = t["fetch_size_kib_per_launch"] * 1024 * t["scale_fetch"] + \
        t["write_size_kib_per_launch"] * 1024 * t["scale_write"]
    assert abs(got - t["bytes_per_launch"]) <= 2
    current = bench.kernel_sources_sha256(srcs) == t["kernel_src_sha256"]
    want = t["bytes_per_launch"] if current else None
    assert bench.measured_traffic("packed", E256, "gather") == want
    assert bench.measured_traffic("packed", E256, "copy") is None
    assert bench.measured_traffic("packed", C.CONFIGS[1].name, "gather") is None
    # a summary taken on other kernel sources is not used
    stale = dict(t, kernel_src_sha256="0" * 64)
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(stale))
    monkeypatch.setitem(bench.FFN_KERNELS, "packed", (str(p), srcs, name))
    assert bench.measured_traffic("packed", E256, "gather") is None


def test_a_failing_variant_is_recorded_not_raised(monkeypatch):
    """The variants run after the line's own measurement: an error in one of
    them is written into the record and the line is still printed."""
    def boom(*a, **k):
        raise RuntimeError("variant failed")

    monkeypatch.setattr(bench, "run_forward", boom)
    monkeypatch.setattr(bench, "prepare", boom)
    a = bench.parse([])
    out = bench.time_variants(C.BY_NAME[E256], a, None, None)
    assert set(out) == {"fp8_first_gemm", "expert_waves"}
    assert all("variant failed" in v["error"] for v in out.values())
    # the fp32 workload has no bf16 variants
    assert bench.time_variants(C.CONFIGS[0], a, None, None) == {}
