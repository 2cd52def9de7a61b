"""The C ABI without a GPU: the library loads, exports everything the header
declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

from top_routing_expert_amd import binding as B
from top_routing_expert_amd import configs as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(moe_\w+)\s*\(", src, flags=re.M)))


def test_header_declarations_match_binding():
    names = _declared_functions()
    assert names == sorted(B.EXPORTS), names


def test_library_exports_every_declared_symbol():
    L = B.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name


def _declared_param_counts():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    out = {}
    for m in re.finditer(r"\b(moe_\w+)\s*\(([^;{]*?)\)\s*;", src):
        params = [p for p in m.group(2).split(",") if p.strip() and p.strip() != "void"]
        out[m.group(1)] = len(params)
    return out


def test_binding_declares_every_signature():
    """Without argtypes ctypes would pass device pointers as 32-bit ints."""
    L = B.lib()
    counts = _declared_param_counts()
    for name in B.EXPORTS:
        f = getattr(L, name)
        assert f.argtypes is not None, name
        assert len(f.argtypes) == counts[name], (name, len(f.argtypes), counts[name])


def test_strerror():
    assert B.strerror(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert B.strerror(s) and B.strerror(s) != "ok"
    assert B.strerror(12345) == "unknown status"


@pytest.mark.parametrize("shape", C.CONFIGS, ids=lambda s: s.name)
def test_workload_configs_are_valid(shape):
    assert B.validate(B.config(shape)) == B.MOE_OK


BAD = [
    (dict(k=0), B.MOE_EINVAL),
    (dict(k=9), B.MOE_EINVAL),            # k > E (E = 8)
    (dict(T=-1), B.MOE_EINVAL),
    (dict(d=0), B.MOE_EINVAL),
    (dict(dtype=7), B.MOE_EINVAL),
    (dict(presel=1), B.MOE_EINVAL),       # presel < k
    (dict(presel=9), B.MOE_EINVAL),       # presel > E
    (dict(n_group=3), B.MOE_EINVAL),      # does not divide E
    (dict(n_group=4, topk_group=0), B.MOE_EINVAL),
    (dict(n_group=4, topk_group=5), B.MOE_EINVAL),
    (dict(n_group=8, topk_group=1), B.MOE_EINVAL),  # 1 group of 1 expert < k
    (dict(renorm=2), B.MOE_EINVAL),
    (dict(ep_ranks=3), B.MOE_EINVAL),     # does not divide E
    (dict(ep_ranks=0), B.MOE_EINVAL),
    (dict(d=4100), B.MOE_EUNSUPPORTED),   # bf16 needs d % 64 == 0
    (dict(f=11000), B.MOE_EUNSUPPORTED),
    (dict(E=2048, k=2), B.MOE_EUNSUPPORTED),
    (dict(k=17, E=64), B.MOE_EUNSUPPORTED),
    (dict(T=1 << 20, d=4096), B.MOE_EUNSUPPORTED),  # (T*k)*max(d,f) >= 2^31
    # (T*k)*max(d,f) = 2^64 would wrap in 64-bit arithmetic
    (dict(T=1 << 30, k=8, E=8, d=1 << 30, f=64), B.MOE_EUNSUPPORTED),
]


@pytest.mark.parametrize("over,want", BAD, ids=[str(b[0]) for b in BAD])
def test_bad_config_rejected_before_launch(over, want):
    cfg = B.config(C.E8_D4096, **over)
    assert B.validate(cfg) == want
    L = B.lib()
    # every routing entry point refuses it without touching any pointer
    assert L.moe_route(ctypes.byref(cfg), None, None, None, None, None, None, None, 0, None) == want
    assert L.moe_permute(ctypes.byref(cfg), None, None, None, None, None, None, None, None, 0,
                         None) == want
    assert L.moe_layer_fwd(ctypes.byref(cfg), None, None, None, None, None, None, None, None, None,
                           0, None) == want


def test_null_config_and_pointers_rejected():
    L = B.lib()
    assert L.moe_validate(None) == B.MOE_EINVAL
    cfg = B.config(C.E8_D4096)
    fake = 1 << 40  # never dereferenced: checks fail first
    # missing outputs / inputs
    assert L.moe_route(ctypes.byref(cfg), fake, fake, None, None, fake, fake, fake, 1 << 30,
                       None) == B.MOE_EINVAL
    assert L.moe_combine(ctypes.byref(cfg), fake, None, fake, fake, None) == B.MOE_EINVAL
    assert L.moe_grouped_ffn(ctypes.byref(cfg), fake, fake, fake, fake, None, fake, fake,
                             None) == B.MOE_EINVAL
    assert L.moe_ffn_gate_up(ctypes.byref(cfg), fake, None, fake, fake, fake, None) == B.MOE_EINVAL
    assert L.moe_ffn_down(ctypes.byref(cfg), fake, fake, fake, None, None) == B.MOE_EINVAL


def test_workspace_too_small_rejected():
    L = B.lib()
    cfg = B.config(C.E8_D4096)
    need = B.workspace_bytes(cfg, "permute")
    assert need > 0
    fake = 1 << 40
    assert L.moe_permute(ctypes.byref(cfg), fake, fake, fake, fake, fake, fake, fake, fake,
                         need - 1, None) == B.MOE_EINVAL
    assert L.moe_permute(ctypes.byref(cfg), fake, fake, fake, fake, fake, fake, fake, fake + 8,
                         need, None) == B.MOE_EINVAL  # misaligned workspace
    lay = B.workspace_bytes(cfg, "layer")
    assert L.moe_layer_fwd(ctypes.byref(cfg), fake, fake, None, fake, fake, fake, fake, None, fake,
                           lay - 1, None) == B.MOE_EINVAL


def test_workspace_sizes():
    for shape in C.CONFIGS:
        cfg = B.config(shape)
        A = shape.T * shape.k
        es = 2 if shape.dtype == "bf16" else 4
        lay = B.workspace_bytes(cfg, "layer")
        # at least the three activation buffers plus the index arrays
        assert lay >= A * (2 * shape.d + shape.f) * es + 4 * A * 4
        assert B.workspace_bytes(cfg, "ffn") == 0
        assert B.workspace_bytes(cfg, "combine") == 0
        assert B.workspace_bytes(cfg, "permute") >= 4 * A
    assert B.workspace_bytes(B.config(C.E8_D4096, T=0), "permute") == 0
    with pytest.raises(B.MoEError):
        B.workspace_bytes(B.config(C.E8_D4096, k=0), "layer")


def test_backward_entries_reject_before_launch():
    """Every backward entry point checks its arguments on the host and
    returns before anything reaches a GPU (so these run without one)."""
    L = B.lib()
    fake = 1 << 40  # 16-byte aligned, never dereferenced
    cfg = B.config(C.E8_D4096)
    f32 = B.config(C.TINY_F32)
    bf = ctypes.byref
    # combine backward
    assert L.moe_combine_backward(bf(f32), fake, fake, fake, fake, fake, fake,
                                  None) == B.MOE_EUNSUPPORTED
    assert L.moe_combine_backward(bf(cfg), None, fake, fake, fake, fake, fake,
                                  None) == B.MOE_EINVAL
    assert L.moe_combine_backward(bf(cfg), fake + 2, fake, fake, fake, fake, fake,
                                  None) == B.MOE_EINVAL  # misaligned rows
    # FFN backward
    need = B.workspace_bytes(cfg, "ffn_backward")
    A, f = C.E8_D4096.T * C.E8_D4096.k, C.E8_D4096.f
    assert need >= 5 * A * f * 2  # a, u, dh / h, da | du
    args = [fake, fake, fake, fake, fake]  # x_perm, offsets, w_gate, w_up, w_down
    outs = [fake, fake, fake, fake, fake]  # d_y_perm, d_x_perm, d_w_gate, d_w_up, d_w_down
    assert L.moe_ffn_backward(bf(f32), *args, None, None, None, None, *outs, fake, 1 << 34,
                              None) == B.MOE_EUNSUPPORTED
    assert L.moe_ffn_backward(bf(cfg), *args, fake, None, None, None, *outs, fake, need,
                              None) == B.MOE_EINVAL  # a without u
    assert L.moe_ffn_backward(bf(cfg), *args, None, None, None, None, *outs, fake, need - 1,
                              None) == B.MOE_EINVAL  # workspace too small
    assert L.moe_ffn_backward(bf(cfg), *args, None, None, None, None, *outs, fake + 16, need,
                              None) == B.MOE_EINVAL  # workspace not 256-byte aligned
    assert L.moe_ffn_backward(bf(cfg), *args, None, None, fake + 2, None, *outs, fake, need,
                              None) == B.MOE_EINVAL  # misaligned packed image
    # packed transposed images for the backward
    dh_b, dx_b = B.packed_weight_bytes_backward(cfg)
    assert dh_b >= C.E8_D4096.E * C.E8_D4096.f * C.E8_D4096.d * 2
    assert dx_b >= C.E8_D4096.E * 2 * C.E8_D4096.f * C.E8_D4096.d * 2
    assert L.moe_pack_weights_backward(bf(f32), fake, fake, fake, fake, fake,
                                       None) == B.MOE_EUNSUPPORTED
    assert L.moe_pack_weights_backward(bf(cfg), fake, fake, fake, None, None,
                                       None) == B.MOE_EINVAL  # no output
    assert L.moe_pack_weights_backward(bf(cfg), fake, fake, None, fake, None,
                                       None) == B.MOE_EINVAL  # dh image without w_down
    assert L.moe_pack_weights_backward(bf(cfg), None, fake, fake, None, fake,
                                       None) == B.MOE_EINVAL  # dx image without w_gate
    # router backward
    rneed = B.workspace_bytes(cfg, "route_backward")
    assert rneed > 0
    rargs = [fake] * 6 + [fake, fake, fake, None]  # ... d_logits, d_x_router, d_w_router, d_bias
    assert L.moe_route_backward(bf(B.config(C.E8_D4096, E=12)), *rargs, fake, 1 << 34,
                                None) == B.MOE_EUNSUPPORTED  # E % 8 != 0
    grouped_presel = B.config(C.E8_D4096, E=16, presel=4, renorm=0, n_group=4, topk_group=2)
    assert L.moe_validate(bf(grouped_presel)) == B.MOE_OK
    assert L.moe_route_backward(bf(grouped_presel), *rargs, fake, 1 << 34,
                                None) == B.MOE_EUNSUPPORTED
    assert L.moe_route_backward(bf(cfg), *rargs, fake, rneed - 1, None) == B.MOE_EINVAL
    # dispatch backward and the training forward
    assert L.moe_unpermute_backward(bf(cfg), fake, fake, fake + 4, fake, None) == B.MOE_EINVAL
    assert L.moe_ffn_gate_up_packed_train(bf(cfg), fake, None, fake, fake, fake, None, fake,
                                          None) == B.MOE_EINVAL  # a missing


C_PROGRAM = r"""
#include <stdio.h>
#include "moe.h"
int main(void) {
  moe_config c = {1024, 4096, 8, 2, 11008, 1, 1, 0, 1, 2, MOE_BF16};
  size_t perm = 0, layer = 0, bwd = 0;
  int s1 = moe_workspace_bytes(&c, MOE_ENTRY_PERMUTE, &perm);
  int s2 = moe_workspace_bytes(&c, MOE_ENTRY_LAYER, &layer);
  int s3 = moe_workspace_bytes(&c, MOE_ENTRY_FFN_BACKWARD, &bwd);
  moe_config bad = c;
  bad.k = 0;
  printf("%d %d %d %zu %zu %zu %d %d %s\n", s1, s2, s3, perm, layer, bwd, moe_validate(&c),
         moe_validate(&bad), moe_strerror(MOE_EUNSUPPORTED));
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_is_a_plain_c_abi(tmp_path):
    """A C99 program (gcc -std=c99 -pedantic -Werror) includes the header,
    links the library and gets the same answers as the Python binding from
    the host-only entry points."""
    src = tmp_path / "t.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "t"
    libdir = os.path.dirname(B.LIB_PATH)
    inc = os.path.join(os.path.dirname(libdir), "include")
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", f"-I{inc}",
                        str(src), f"-L{libdir}", "-lmoe_mi355x", f"-Wl,-rpath,{libdir}", "-o",
                        str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr[-2000:]
    f = r.stdout.split(maxsplit=8)
    cfg = B.config(C.E8_D4096)
    assert [int(v) for v in f[:3]] == [B.MOE_OK] * 3
    assert int(f[3]) == B.workspace_bytes(cfg, "permute")
    assert int(f[4]) == B.workspace_bytes(cfg, "layer")
    assert int(f[5]) == B.workspace_bytes(cfg, "ffn_backward")
    assert int(f[6]) == B.MOE_OK and int(f[7]) == B.MOE_EINVAL
    assert f[8].strip() == B.strerror(B.MOE_EUNSUPPORTED)


def test_noalloc_permute_rejects_beyond_its_scratch_before_launch():
    """moe_permute_noalloc checks its scratch need against the static array on
    the host (4 (ceil(T/256) E + T k) bytes > 16 MiB here) before any HIP call."""
    L = B.lib()
    assert L.moe_noalloc_scratch_bytes() == 16 << 20
    cfg = B.config(C.E8_D4096.replace(T=1 << 20, k=8, d=64, f=64))
    fake = ctypes.c_void_p(256)
    st = L.moe_permute_noalloc(ctypes.byref(cfg), None, fake, fake, fake, fake, fake, None, None)
    assert st == B.MOE_ESCRATCH
    bad = B.config(C.E8_D4096.replace(k=0))
    assert L.moe_permute_noalloc(ctypes.byref(bad), None, fake, fake, fake, fake, fake, None,
                                 None) == B.MOE_EINVAL


def test_fp8_gemm_entries_reject_before_launch():
    """The FP8 first GEMM takes bf16 problems with d a multiple of 128 only,
    and checks its pointers and alignments on the host."""
    L = B.lib()
    fake = ctypes.c_void_p(4096)
    n = ctypes.c_size_t(0)
    ok = B.config(C.E8_D4096.replace(d=256, f=128))
    assert L.moe_fp8_weight_bytes(ctypes.byref(ok), ctypes.byref(n)) == B.MOE_OK and n.value > 0
    for bad, want in ((C.E8_D4096.replace(d=192), B.MOE_EUNSUPPORTED),
                      (C.TINY_F32, B.MOE_EUNSUPPORTED)):
        cfg = B.config(bad)
        assert L.moe_fp8_weight_bytes(ctypes.byref(cfg), ctypes.byref(n)) == want
        assert L.moe_pack_weights_fp8(ctypes.byref(cfg), fake, fake, fake, None) == want
        assert L.moe_ffn_gate_up_fp8_gather(ctypes.byref(cfg), fake, fake, fake, fake, fake, fake,
                                            None) == want
    assert L.moe_fp8_weight_bytes(ctypes.byref(ok), None) == B.MOE_EINVAL
    assert L.moe_pack_weights_fp8(ctypes.byref(ok), fake, None, fake, None) == B.MOE_EINVAL
    assert L.moe_pack_weights_fp8(ctypes.byref(ok), fake, fake, ctypes.c_void_p(4096 + 16),
                                  None) == B.MOE_EINVAL  # image not 256-byte aligned
    assert L.moe_ffn_gate_up_fp8_gather(ctypes.byref(ok), fake, fake, None, fake, fake, fake,
                                        None) == B.MOE_EINVAL


def test_waved_layer_rejects_before_launch():
    """Wave counts that do not divide E, a caller x_perm (the waves gather
    their rows) and fp32 problems are refused on the host."""
    L = B.lib()
    fake = ctypes.c_void_p(4096)
    cfg = B.config(C.SMALL["e8"])
    bufs = B.MoELayerBufs(x_perm=4096)
    for n_waves, b in ((0, None), (3, None), (16, None), (2, ctypes.byref(bufs))):
        assert L.moe_layer_fwd_packed_waved(ctypes.byref(cfg), fake, fake, None, fake, fake, fake,
                                            b, fake, 1 << 30, n_waves, None, None) == B.MOE_EINVAL
    f32 = B.config(C.TINY_F32)
    assert L.moe_layer_fwd_packed_waved(ctypes.byref(f32), fake, fake, None, fake, fake, fake,
                                        None, fake, 1 << 30, 2, None, None) == B.MOE_EUNSUPPORTED
