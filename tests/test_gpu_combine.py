"""Combine parity against the oracle, and the identity-expert composition
combine(permute(x)) = x (renormalised gates)."""
import numpy as np
import pytest
import torch

from _gpu import TOL_STAGE, host, log, rel_err
from oracle import moe_oracle as om
from top_routing_expert_amd import binding as B
from top_routing_expert_amd import configs as C
from top_routing_expert_amd import inputs as I

pytestmark = pytest.mark.gpu

CASES = [(1, 64, 8, 2, "bf16"), (1000, 256, 64, 2, "bf16"), (333, 512, 256, 8, "bf16"),
         (77, 128, 1024, 16, "bf16"), (130, 320, 12, 3, "bf16"), (500, 192, 16, 4, "bf16"),
         (256, 64, 8, 2, "f32"), (129, 68, 8, 3, "f32")]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_combine_matches_oracle(case):
    T, d, E, k, dtype = case
    log(f"[combine] {case}")
    rng = np.random.default_rng(T + d)
    shape = C.E8_D4096.replace(name="comb", T=T, d=d, E=E, k=k, dtype=dtype, ep_ranks=1)
    A = T * k
    y_np = I.make_x(shape.replace(T=A), seed=15)
    slot_np = rng.permutation(A).astype(np.int32)
    w_np = rng.random((T, k)).astype(np.float32)
    y, slot, w = B.to_device(y_np), torch.from_numpy(slot_np).cuda(), torch.from_numpy(w_np).cuda()
    out = torch.empty((T, d), dtype=y.dtype, device="cuda")
    B.moe_combine(B.config(shape), y, slot, w, out)
    torch.cuda.synchronize()
    want = om.combine(y_np, slot_np, w_np)
    assert rel_err(host(out), want) <= TOL_STAGE[dtype]


@pytest.mark.parametrize("k", [1, 2, 8])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_identity_experts_give_back_x(k, dtype):
    """With y_perm = x_perm and renormalised gates, out = x * sum(g) = x."""
    log(f"[combine] identity k={k} {dtype}")
    T, d, E = 600, 128, 16
    shape = C.E8_D4096.replace(name="ident", T=T, d=d, E=E, k=k, dtype=dtype, ep_ranks=4,
                               presel=0, renorm=1)
    cfg = B.config(shape)
    rng = np.random.default_rng(k)
    x_np = I.make_x(shape, seed=16)
    logits = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).cuda()
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    B.moe_route(cfg, None, None, None, logits, idx, w)
    x = B.to_device(x_np)
    A = T * k
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    roffs = torch.empty(5, dtype=torch.int32, device="cuda")
    slot = torch.empty(A, dtype=torch.int32, device="cuda")
    src = torch.empty(A, dtype=torch.int32, device="cuda")
    xp = torch.empty((A, d), dtype=x.dtype, device="cuda")
    B.moe_permute(cfg, x, idx, offs, roffs, slot, src, xp, B.workspace(cfg, "permute"))
    out = torch.empty_like(x)
    B.moe_combine(cfg, xp, slot, w, out)
    torch.cuda.synchronize()
    if dtype == "bf16" or k == 1:
        # x * (1 +- a few fp32 ulps) rounds back to the same bf16 value; k = 1 is exact
        assert np.array_equal(host(out), x_np)
    else:
        assert np.max(np.abs(host(out) - x_np) / np.maximum(np.abs(x_np), 1e-30)) <= 4 * 2.0 ** -23
