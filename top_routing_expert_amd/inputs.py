"""Seeded synthetic inputs, shared by the tests, the bench and the smoke check.

Recipe (the same for every shape):
  * x ~ N(0, x_std^2), router / gate / up / down weights ~ N(0, w_std^2), drawn in
    float32 and, for bf16 shapes, rounded to bfloat16 (round to nearest even).
  * bias: "normal" draws b_e ~ N(0,1); "zipf" sets b_e = -1.1*ln(e+1), the log
    of a Zipf(1.1) prior with expert 0 hottest; "none" gives no bias.
  * Every tensor draws from its own numpy PCG64 stream keyed by
    SeedSequence([seed, tensor_id, part]); tensor ids are 0 x, 1 router,
    2 bias, 3 gate, 4 up, 5 down; `part` is the expert for expert weights and
    the 1024-row block for x, so large tensors are generated in parallel.

bf16 tensors are held as uint16 bit patterns.  This module contains no step of
the MoE computation itself.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

from .configs import MoEShape

TID_X, TID_ROUTER, TID_BIAS, TID_GATE, TID_UP, TID_DOWN, TID_DOUT = range(7)
X_BLOCK_ROWS = 1024


def _rng(seed: int, tid: int, part: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, part])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_block(seed, tid, part, shape, std, bf16):
    a = _rng(seed, tid, part).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return f32_to_bf16_bits(a) if bf16 else a


def make_bias(shape: MoEShape, seed: int) -> np.ndarray | None:
    if shape.bias == "none":
        return None
    if shape.bias == "normal":
        return _rng(seed, TID_BIAS, 0).standard_normal(shape.E, dtype=np.float32)
    if shape.bias == "zipf":
        return (-1.1 * np.log(np.arange(shape.E, dtype=np.float64) + 1.0)).astype(np.float32)
    raise ValueError(f"unknown bias kind {shape.bias!r}")


def make_x(shape: MoEShape, seed: int, pool=None) -> np.ndarray:
    bf16 = shape.dtype == "bf16"
    out = np.empty((shape.T, shape.d), dtype=np.uint16 if bf16 else np.float32)

    def blk(b):
        r0 = b * X_BLOCK_ROWS
        r1 = min(shape.T, r0 + X_BLOCK_ROWS)
        out[r0:r1] = _normal_block(seed, TID_X, b, (r1 - r0, shape.d), shape.x_std, bf16)

    nb = (shape.T + X_BLOCK_ROWS - 1) // X_BLOCK_ROWS
    _run(pool, blk, range(nb))
    return out


def make_expert_weight(shape: MoEShape, seed: int, tid: int, pool=None) -> np.ndarray:
    """[E, rows, cols] with (rows, cols) = (f, d) for gate/up and (d, f) for down."""
    bf16 = shape.dtype == "bf16"
    rc = (shape.f, shape.d) if tid in (TID_GATE, TID_UP) else (shape.d, shape.f)
    out = np.empty((shape.E,) + rc, dtype=np.uint16 if bf16 else np.float32)

    def one(e):
        out[e] = _normal_block(seed, tid, e, rc, shape.w_std, bf16)

    _run(pool, one, range(shape.E))
    return out


def make_grad_out(shape: MoEShape, seed: int) -> np.ndarray:
    """The gradient arriving at the layer's output for a backward step: [T, d]
    standard normal (bf16 bits for bf16 shapes)."""
    return _normal_block(seed, TID_DOUT, 0, (shape.T, shape.d), 1.0, shape.dtype == "bf16")


def make_router(shape: MoEShape, seed: int) -> np.ndarray:
    return _normal_block(seed, TID_ROUTER, 0, (shape.E, shape.d), shape.w_std,
                         shape.dtype == "bf16")


def _run(pool, fn, items):
    items = list(items)
    if pool is None and len(items) > 1:
        with cf.ThreadPoolExecutor(_threads()) as p:
            list(p.map(fn, items))
    elif pool is not None:
        list(pool.map(fn, items))
    else:
        for i in items:
            fn(i)


def make_inputs(shape: MoEShape, seed: int, with_experts: bool = True) -> dict:
    """All inputs of one MoE layer forward, as numpy arrays (bf16 as uint16 bits)."""
    with cf.ThreadPoolExecutor(_threads()) as pool:
        d = {
            "x": make_x(shape, seed, pool),
            "w_router": make_router(shape, seed),
            "bias": make_bias(shape, seed),
        }
        if with_experts:
            d["w_gate"] = make_expert_weight(shape, seed, TID_GATE, pool)
            d["w_up"] = make_expert_weight(shape, seed, TID_UP, pool)
            d["w_down"] = make_expert_weight(shape, seed, TID_DOWN, pool)
    return d
