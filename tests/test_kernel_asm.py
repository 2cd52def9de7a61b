"""Static checks of the packed grouped-GEMM kernels' machine code (CPU only).

The main loop loads weight fragments with asynchronous asm loads and waits for
them with explicit counts.  The compiler treats an asm output as available as
soon as the asm statement issues, so the code is only correct if the compiler
never copies, spills or overwrites such a register before the explicit wait
(only the matrix instructions after the wait may read it).  This compiles the
kernel source to gfx950 assembly and checks exactly that."""
import os
import re
import shutil
import subprocess

import pytest

from top_routing_expert_amd import build as Bld

# (source file, kernel-name substring) of every kernel with asynchronous asm loads
ASYNC_KERNELS = [("ffn_packed.hip", "gemm_packed"), ("route.hip", "router_skinny")]


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {tok} if re.match(r"[va]\d+$", tok) else set()


def _kernel_bodies(asm: str, kernel_pat: str):
    """(name, instruction lines) of every kernel whose symbol matches."""
    out, body, name = [], None, None
    for line in asm.split("\n"):
        if re.match(r"^_Z\w*:", line) and kernel_pat in line:
            body, name = [], line
            continue
        if body is None:
            continue
        body.append(line)
        if "s_endpgm" in line:
            out.append((name, body))
            body = None
    return out


def _blocks(lines):
    """Basic blocks of a kernel body: list of (label, instructions, successor
    labels).  A block ends at a label or after a branch / s_endpgm."""
    blocks, cur, label = [], [], "entry"
    n = 0

    def close(succ):
        nonlocal cur, label, n
        blocks.append([label, cur, succ])
        n += 1
        cur, label = [], f"_fall{n}"

    for line in lines:
        m = re.match(r"^(\.\w+):", line)
        if m:
            close([m.group(1)])  # falls through into the label (may be empty)
            label = m.group(1)
            continue
        cur.append(line)
        ins = line.strip().split(";")[0].strip()
        op = ins.split()[0] if ins else ""
        if op == "s_branch":
            close([ins.split()[1]])
        elif op.startswith("s_cbranch"):
            close([ins.split()[1], f"_fall{n + 1}"])
        elif op == "s_endpgm":
            close([])
    if cur:
        close([])
    return blocks


def _transfer(lines, pending, report):
    """Walk one block: returns the pending set at its end; report(ins) for
    every non-asm instruction that touches a pending register."""
    in_asm = False
    pending = set(pending)
    for line in lines:
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        ins = s.split(";")[0].strip()
        if not ins or ins.startswith("."):
            continue
        op = ins.split()[0]
        args = [a.strip() for a in ins[len(op):].split(",")]
        if in_asm:
            if op == "buffer_load_dwordx4" and " lds" not in ins:
                pending |= _regs(args[0])
            elif op == "s_waitcnt" and "vmcnt" in ins:
                pending = set()
            continue
        if op == "s_waitcnt" and "vmcnt(0)" in ins:
            pending = set()
            continue
        if not pending or op.startswith("v_mfma"):
            continue
        touched = set()
        for a in args:
            touched |= _regs(a.split()[0] if a else "")
        if touched & pending:
            report(ins)
    return pending


def in_flight_violations(asm: str, kernel_pat: str = "gemm_packed"):
    """(kernel, instruction) pairs that read or write a register whose async
    asm load has not been waited for on some path through the kernel's
    control flow (any explicit asm vmcnt wait counts as waiting for all of
    them: the waits' counts are checked by the schedule, this checks that
    the compiler leaves the registers alone in between)."""
    out = []
    for name, lines in _kernel_bodies(asm, kernel_pat):
        blocks = _blocks(lines)
        index = {b[0]: k for k, b in enumerate(blocks)}
        entry_in = [set() for _ in blocks]
        work = list(range(len(blocks)))
        while work:
            k = work.pop(0)
            end = _transfer(blocks[k][1], entry_in[k], lambda ins: None)
            for t in blocks[k][2]:
                if t in index:
                    q = index[t]
                    if not end <= entry_in[q]:
                        entry_in[q] |= end
                        work.append(q)
        seen = set()
        for k, b in enumerate(blocks):
            def rep(ins):
                if ins not in seen:
                    seen.add(ins)
                    out.append((name, ins))
            _transfer(b[1], entry_in[k], rep)
    return out


def test_checker_flags_a_copy_of_an_in_flight_register():
    asm = "\n".join([
        "_Zgemm_packed_k:",
        ";;#ASMSTART", "buffer_load_dwordx4 v[4:7], v1, s[0:3], s4 offen offset:0", ";;#ASMEND",
        "v_mov_b32 v20, v5",
        ";;#ASMSTART", "s_waitcnt vmcnt(0)", ";;#ASMEND",
        "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]",
        "s_endpgm",
    ])
    assert len(in_flight_violations(asm)) == 1
    ok = asm.replace("v_mov_b32 v20, v5", "v_mov_b32 v20, v9")
    assert in_flight_violations(ok) == []


def test_checker_follows_control_flow():
    load = [";;#ASMSTART", "buffer_load_dwordx4 v[4:7], v1, s[0:3], s4 offen offset:0", ";;#ASMEND"]
    wait = [";;#ASMSTART", "s_waitcnt vmcnt(0)", ";;#ASMEND"]
    # the load at the bottom of a loop is still in flight at its top
    loop = "\n".join(["_Zgemm_packed_k:", ".LBB0_1:", "v_mov_b32 v20, v5", *wait,
                      "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]", *load,
                      "s_cbranch_scc1 .LBB0_1", "s_endpgm"])
    assert len(in_flight_violations(loop)) == 1
    # ... and at the target of a conditional branch's fall-through label
    fall = "\n".join(["_Zgemm_packed_k:", *load, "s_cbranch_scc1 .LBB0_2", ".LBB0_3:",
                      "v_mov_b32 v20, v6", ".LBB0_2:", *wait, "s_endpgm"])
    assert len(in_flight_violations(fall)) == 1
    # a block after an unconditional branch is not reached from the load
    other = "\n".join(["_Zgemm_packed_k:", *load, *wait, "s_branch .LBB0_4", *load,
                       "s_branch .LBB0_5", ".LBB0_6:", "v_mov_b32 v20, v6", ".LBB0_5:", *wait,
                       ".LBB0_4:", "s_endpgm"])
    assert in_flight_violations(other) == []


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
@pytest.mark.parametrize("src,kernel", ASYNC_KERNELS, ids=[k for _, k in ASYNC_KERNELS])
def test_kernel_never_touches_in_flight_load_registers(tmp_path, src, kernel):
    out = tmp_path / (src + ".s")
    cmd = [Bld._hipcc(), *Bld.HIPCC_FLAGS, "--cuda-device-only", "-S",
           os.path.join(Bld.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    assert asm.count("buffer_load_dwordx4") > 0
    bad = in_flight_violations(asm, kernel)
    assert bad == [], bad[:5]
    # no scratch: every spill would be a chance for the above
    assert not re.search(r"\.private_segment_fixed_size:\s+[1-9]", asm)


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_fp8_decode_rounds_twice(tmp_path):
    """The receiver's decode is code * s, rounded, then + z, rounded (two
    float32 roundings, as the oracle computes it).  A fused multiply-add
    rounds once and changes some decoded rows, so the decode kernel's machine
    code must hold no fma at all (the quantiser's fmas are those of the IEEE
    division sequence, which is correctly rounded)."""
    out = tmp_path / "fp8.s"
    cmd = [Bld._hipcc(), *Bld.HIPCC_FLAGS, "--cuda-device-only", "-S",
           os.path.join(Bld.CSRC, "fp8.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()

    def whole_bodies(pat):  # up to the function's end label (early returns end in s_endpgm too)
        return [(m.group(1), m.group(2).split("\n"))
                for m in re.finditer(r"^(_Z\w*" + pat + r"\w*):[^\n]*\n(.*?)^\.Lfunc_end", asm, re.M | re.S)]

    bodies = whole_bodies("fp8_dequantize_gather_kernel")
    assert len(bodies) >= 1
    for _, lines in bodies:
        body = "\n".join(lines)
        assert re.search(r"v_mul_f32", body) and re.search(r"v_add_f32", body)
        assert not re.search(r"v_(pk_)?fmac?_", body)
    q = whole_bodies("fp8_quantize_rows_kernel")
    assert len(q) >= 1
    for _, lines in q:
        # every fma there sits between a v_div_scale and its v_div_fixup
        in_div = False
        for line in lines:
            if "v_div_scale_f32" in line:
                in_div = True
            if re.search(r"v_(pk_)?fmac?_", line):
                assert in_div, line
            if "v_div_fixup_f32" in line:
                in_div = False
        assert "v_div_fixup_f32" in "\n".join(lines)


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_backward_kernels_keep_everything_in_registers(tmp_path):
    """The backward GEMMs hold up to 256 registers per lane; a spill would put
    scratch traffic into their main loops."""
    out = tmp_path / "backward.s"
    cmd = [Bld._hipcc(), *Bld.HIPCC_FLAGS, "--cuda-device-only", "-S",
           os.path.join(Bld.CSRC, "backward.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    meta = out.read_text().split("amdhsa.kernels", 1)[1]
    kernels = re.findall(r"\.name:\s+(\S+)[\s\S]*?\.private_segment_fixed_size:\s+(\d+)", meta)
    assert any("dgrad_dma_kernel" in n for n, _ in kernels)
    assert any("wgrad_dma_kernel" in n for n, _ in kernels)
    assert [n for n, ps in kernels if int(ps)] == []
