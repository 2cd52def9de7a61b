"""Dispatch-layout parity: offsets, rank offsets, slot_of and src_of must be
bit-exact against the oracle; x_perm rows must be bitwise copies of their
source rows."""
import numpy as np
import pytest
import torch

from _gpu import host, log
from oracle import moe_oracle as om
from top_routing_expert_amd import binding as B
from top_routing_expert_amd import configs as C
from top_routing_expert_amd import inputs as I

pytestmark = pytest.mark.gpu


def _topk(kind, T, E, k, rng):
    if kind == "random":
        return np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    if kind == "hot":  # every token picks the same k experts: one segment per expert of T rows
        return np.tile(np.arange(k, dtype=np.int32)[::-1], (T, 1))
    if kind == "skew":  # Zipf-like preference, expert 0 hottest, many experts empty
        p = 1.0 / np.arange(1, E + 1) ** 2.0
        out = np.empty((T, k), np.int32)
        for t in range(T):
            out[t] = rng.choice(E, size=k, replace=False, p=p / p.sum())
        return out
    raise ValueError(kind)


def _run(shape, x_np, idx_np):
    cfg = B.config(shape)
    A = shape.T * shape.k
    x = B.to_device(x_np)
    idx = torch.from_numpy(idx_np).cuda()
    offs = torch.full((shape.E + 1,), -7, dtype=torch.int32, device="cuda")
    roffs = torch.full((shape.ep_ranks + 1,), -7, dtype=torch.int32, device="cuda")
    slot = torch.empty(A, dtype=torch.int32, device="cuda")
    src = torch.empty(A, dtype=torch.int32, device="cuda")
    xp = torch.empty((A, shape.d), dtype=x.dtype, device="cuda")
    B.moe_permute(cfg, x, idx, offs, roffs, slot, src, xp, B.workspace(cfg, "permute"))
    torch.cuda.synchronize()
    return x, offs, roffs, slot, src, xp


def _check(shape, idx_np, x, offs, roffs, slot, src, xp):
    o = om.permute(idx_np, shape.E, shape.ep_ranks)
    assert np.array_equal(host(offs), o["offsets"])
    assert np.array_equal(host(roffs), o["rank_offsets"])
    assert np.array_equal(host(slot), o["slot_of"])
    assert np.array_equal(host(src), o["src_of"])
    # bitwise row copies, checked on the device with torch indexing
    src_rows = torch.from_numpy(o["src_of"].astype(np.int64) // shape.k).cuda()
    view = torch.int16 if x.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(xp.view(view), x.view(view)[src_rows])


CASES = [
    # (T, d, E, k, R, dtype, kind)
    (1, 64, 8, 2, 2, "bf16", "random"),
    (255, 128, 8, 2, 2, "bf16", "random"),
    (256, 128, 8, 2, 4, "bf16", "random"),
    (257, 128, 16, 2, 4, "bf16", "random"),
    (1000, 256, 64, 2, 8, "bf16", "skew"),
    (4099, 64, 256, 8, 64, "bf16", "random"),
    (777, 64, 1024, 16, 1024, "bf16", "random"),
    (513, 192, 16, 4, 4, "bf16", "hot"),
    (300, 64, 8, 1, 1, "bf16", "random"),
    (256, 64, 8, 2, 2, "f32", "random"),
    (333, 68, 8, 3, 8, "f32", "skew"),
    # batches of at most 4 chunks of 256 tokens with E <= 256 count and scan
    # in one block; larger ones in two kernels
    (1024, 64, 256, 8, 8, "bf16", "random"),   # 4 chunks, E = 256: one block
    (1025, 64, 8, 2, 2, "bf16", "hot"),        # 5 chunks: two kernels, one token in the last
    (4096, 64, 64, 2, 8, "bf16", "skew"),      # 16 chunks
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_permute_matches_oracle(case):
    T, d, E, k, R, dtype, kind = case
    log(f"[permute] {case}")
    rng = np.random.default_rng(T + E)
    shape = C.E8_D4096.replace(name="perm", T=T, d=d, E=E, k=k, ep_ranks=R, dtype=dtype,
                               f=64, presel=0, renorm=1)
    x_np = I.make_x(shape, seed=3)
    idx_np = _topk(kind, T, E, k, rng)
    _check(shape, idx_np, *_run(shape, x_np, idx_np))


@pytest.mark.parametrize("shape", C.CONFIGS[1:], ids=lambda s: s.name)
def test_permute_full_size(shape):
    log(f"[permute] full {shape.name}")
    rng = np.random.default_rng(shape.E)
    x_np = I.make_x(shape, seed=4)
    idx_np = _topk("random", shape.T, shape.E, shape.k, rng)
    _check(shape, idx_np, *_run(shape, x_np, idx_np))


def test_permute_empty_batch():
    log("[permute] T=0")
    shape = C.E8_D4096.replace(T=0)
    cfg = B.config(shape)
    offs = torch.full((shape.E + 1,), -7, dtype=torch.int32, device="cuda")
    roffs = torch.full((shape.ep_ranks + 1,), -7, dtype=torch.int32, device="cuda")
    B.moe_permute(cfg, None, None, offs, roffs, None, None, None, None)
    torch.cuda.synchronize()
    assert host(offs).tolist() == [0] * (shape.E + 1)
    assert host(roffs).tolist() == [0] * (shape.ep_ranks + 1)


def test_permute_deterministic():
    log("[permute] determinism")
    shape = C.SMALL["e256"]
    rng = np.random.default_rng(5)
    x_np = I.make_x(shape, seed=5)
    idx_np = _topk("random", shape.T, shape.E, shape.k, rng)
    a = [t.cpu() for t in _run(shape, x_np, idx_np)[1:]]
    b = [t.cpu() for t in _run(shape, x_np, idx_np)[1:]]
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.int16) if v.dtype == torch.bfloat16 else v)


@pytest.mark.parametrize("T,E,k", [(1000, 64, 2), (300, 8, 1), (4099, 256, 8)])
def test_permute_indices_only(T, E, k):
    """x and x_perm NULL: the same index outputs, no row copies."""
    log(f"[permute] indices only T={T} E={E} k={k}")
    rng = np.random.default_rng(T + E)
    shape = C.E8_D4096.replace(name="perm-idx", T=T, d=64, E=E, k=k, ep_ranks=4)
    idx_np = _topk("random", T, E, k, rng)
    x_np = I.make_x(shape, seed=3)
    _, offs, roffs, slot, src, _ = _run(shape, x_np, idx_np)
    cfg = B.config(shape)
    A = T * k
    idx = torch.from_numpy(idx_np).cuda()
    offs2 = torch.full_like(offs, -7)
    roffs2 = torch.full_like(roffs, -7)
    slot2 = torch.full((A,), -7, dtype=torch.int32, device="cuda")
    src2 = torch.full((A,), -7, dtype=torch.int32, device="cuda")
    B.moe_permute(cfg, None, idx, offs2, roffs2, slot2, src2, None, B.workspace(cfg, "permute"))
    torch.cuda.synchronize()
    for a, b in ((offs, offs2), (roffs, roffs2), (slot, slot2), (src, src2)):
        assert torch.equal(a, b)
    # one of x / x_perm alone is rejected
    with pytest.raises(RuntimeError):
        B.moe_permute(cfg, B.to_device(x_np), idx, offs2, roffs2, slot2, src2, None,
                      B.workspace(cfg, "permute"))
