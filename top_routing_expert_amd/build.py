"""Builds libmoe_mi355x.so for gfx950 with hipcc (in-tree, no JIT cache).

Every HIP source under csrc/ is compiled to an object in _build/ (in
parallel), then linked into top_routing_expert_amd/libmoe_mi355x.so.  All
device code is compiled with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_mi355x.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", "-Wno-inline-asm",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False, jobs: int | None = None) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = jobs or min(8, len(srcs))
    with cf.ThreadPoolExecutor(jobs) as pool:
        futs = [pool.submit(_run, [hipcc, *HIPCC_FLAGS, "-c", s, "-o", o]) for s, o in zip(srcs, objs)]
        for f in futs:
            msg = f.result()
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
