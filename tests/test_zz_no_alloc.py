"""moe_permute_noalloc, the permute for callers that cannot allocate: its
scratch is the library's static device array instead of a workspace.  Its
outputs must equal moe_permute's bit for bit, on consecutive calls that
share the array (the second one smaller, so stale values of the first stay
in the array), with and without the row copy."""
import numpy as np
import pytest
import torch

from _gpu import host, log
from top_routing_expert_amd import binding as B
from top_routing_expert_amd import configs as C
from top_routing_expert_amd import inputs as I

pytestmark = pytest.mark.gpu

FIELDS = ("expert_offsets", "rank_offsets", "slot_of", "src_of", "x_perm")


def _buffers(shape, fill):
    T, E, k, d, R = shape.T, shape.E, shape.k, shape.d, shape.ep_ranks
    i32 = torch.int32
    return dict(expert_offsets=torch.full((E + 1,), fill, dtype=i32, device="cuda"),
                rank_offsets=torch.full((R + 1,), fill, dtype=i32, device="cuda"),
                slot_of=torch.full((T * k,), fill, dtype=i32, device="cuda"),
                src_of=torch.full((T * k,), fill, dtype=i32, device="cuda"),
                x_perm=torch.full((T * k, d), fill, dtype=torch.int16,
                                  device="cuda").view(torch.bfloat16))


def _compare(shape, seed, rows=True):
    log(f"[noalloc] {shape.name} T={shape.T} E={shape.E} k={shape.k} rows={rows}")
    rng = np.random.default_rng(seed)
    idx = torch.from_numpy(np.argsort(rng.random((shape.T, shape.E)), axis=1)[:, :shape.k]
                           .astype(np.int32)).cuda()
    x = B.to_device(I.make_x(shape, seed)) if rows else None
    cfg = B.config(shape)
    ref, got = _buffers(shape, 7), _buffers(shape, -5)
    B.moe_permute(cfg, x, idx, ref["expert_offsets"], ref["rank_offsets"], ref["slot_of"],
                  ref["src_of"], ref["x_perm"] if rows else None, B.workspace(cfg, "permute"))
    B.moe_permute_noalloc(cfg, x, idx, got["expert_offsets"], got["rank_offsets"],
                          got["slot_of"], got["src_of"], got["x_perm"] if rows else None)
    torch.cuda.synchronize()
    for n in FIELDS if rows else FIELDS[:-1]:
        assert np.array_equal(host(ref[n]), host(got[n])), n
    if not rows:  # no row copy requested: x_perm untouched
        assert bool((got["x_perm"].view(torch.int16) == -5).all())


BIG = C.E256_GROUPED.replace(name="noalloc-big", d=256)            # 32 chunks x 256 experts
SMALL = C.E8_D4096.replace(name="noalloc-small", T=300, d=64)      # one fused count + scan


def test_noalloc_permute_equals_workspace_permute_on_consecutive_calls():
    assert B.noalloc_scratch_bytes() == 16 << 20
    _compare(BIG, 1)
    _compare(SMALL, 2)             # smaller: the big call's counts and ranks are still there
    _compare(BIG, 3, rows=False)   # index outputs only
    _compare(SMALL.replace(T=1), 4)
    _compare(SMALL.replace(T=0), 5)


def test_noalloc_permute_rejects_problems_beyond_its_scratch():
    shape = C.E8_D4096.replace(name="noalloc-too-big", T=1 << 20, k=8, d=64, f=64)
    cfg = B.config(shape)
    dummy = torch.empty(16, dtype=torch.int32, device="cuda")
    with pytest.raises(B.MoEError) as ei:
        B.moe_permute_noalloc(cfg, None, dummy, dummy, dummy, dummy, dummy, None)
    assert ei.value.status == B.MOE_ESCRATCH
