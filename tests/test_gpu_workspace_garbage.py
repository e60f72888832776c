"""GPU: workspaces need no initialisation.  Route and forward run once with
zero-filled workspaces and once with workspaces full of 0xFF bytes (NaN in
every float view, -1 in every integer view); ids, gates and outputs must be
bitwise equal.  Covers the decode route and GEMV path, the general path,
the many-token bounded router, the fp64 matrix-core router (fp32 inputs, or
a logits output), the prefill matrix-core paths (MXFP4 on the scaled MFMA,
bf16 and NVFP4 on the bf16 MFMA), masked forwards through slot
indirection, and the fused route + forward call (in-kernel selection at one
token, the two-call branch at four)."""
import numpy as np
import pytest
import torch

from gpu_util import LayerData, dev
from sparse_moe_expert_softmax_amd import ftmoe
from sparse_moe_expert_softmax_amd.configs import BF16, C1, C2, C3, C5, MXFP4, NVFP4, MoEConfig

pytestmark = pytest.mark.gpu

MID = MoEConfig("prefill_mid_mxfp4", 91, hidden=512, inter=384, n_experts=16, top_k=4, act_dtype=BF16,
                router_dtype=BF16, w_dtype=MXFP4, n_layers=1)
MID_BF = MoEConfig("prefill_mid_bf16", 131, hidden=512, inter=384, n_experts=16, top_k=4, act_dtype=BF16,
                   router_dtype=BF16, w_dtype=BF16, n_layers=1)
MID_NV = MoEConfig("prefill_mid_nvfp4", 135, hidden=512, inter=384, n_experts=16, top_k=4, act_dtype=BF16,
                   router_dtype=BF16, w_dtype=NVFP4, n_layers=1)


def run(ld, fill, logits=False, mask=None, slots=None):
    cfg, T = ld.cfg, ld.T
    rws = torch.full((max(ftmoe.ft_route_workspace_bytes(ld.desc, T), 256),), fill, dtype=torch.uint8, device="cuda")
    fws = torch.full((max(ftmoe.ft_moe_workspace_bytes(ld.desc, T), 256),), fill, dtype=torch.uint8, device="cuda")
    ids = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, cfg.top_k), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, cfg.n_experts), dtype=torch.float64, device="cuda") if logits else None
    ftmoe.ft_moe_route(ld.desc, dev(ld.x), dev(ld.wr), ids, gates, logits=lg, workspace=rws)
    torch.cuda.synchronize()
    ld.build_pool(ids.cpu().numpy().ravel())
    out = torch.empty((T, cfg.hidden), dtype=torch.float32, device="cuda")
    pool, sl = ld.pool, None
    if slots is not None:  # records moved to other slots, reached through slot_ids
        e_ids = ids.cpu().numpy()
        uniq = sorted(set(e_ids.ravel().tolist()))
        pool = torch.full((2 * len(uniq) + 1, ld.stride), 0xFF, dtype=torch.uint8, device="cuda")
        for i, e in enumerate(uniq):
            pool[2 * i + 1].copy_(ld.pool[e])
        sl = dev(np.vectorize({e: 2 * i + 1 for i, e in enumerate(uniq)}.get)(e_ids).astype(np.int32))
    m = None if mask is None else dev(np.asarray(mask, dtype=np.uint32))
    ftmoe.ft_moe_forward(ld.desc, dev(ld.x), ids, gates, pool, out, fws, slot_ids=sl, expert_mask=m)
    torch.cuda.synchronize()
    return (ids, gates, out) + ((lg,) if logits else ())


@pytest.mark.parametrize("cfg,T", [(C2, 1), (C2, 4), (C2, 17), (C3, 2), (MID, 300), (MID_BF, 300), (MID_NV, 300)])
def test_results_do_not_depend_on_workspace_contents(cfg, T):
    print(f"workspace garbage {cfg.name} T={T}", flush=True)
    ld = LayerData(cfg, 0, 3, T)
    a = run(ld, 0)
    b = run(ld, 0xFF)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    assert not torch.isnan(a[2]).any()


@pytest.mark.parametrize("cfg,T,logits", [(C1, 40, False), (C2, 20, True)])
def test_fp64_matrix_core_router_ignores_workspace_contents(cfg, T, logits):
    """More than 16 tokens with fp32 operands, or with the logits requested,
    run the fp64 matrix-core router."""
    print(f"workspace garbage fp64 router {cfg.name} T={T} logits={logits}", flush=True)
    ld = LayerData(cfg, 0, 4, T)
    a = run(ld, 0, logits=logits)
    b = run(ld, 0xFF, logits=logits)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


@pytest.mark.parametrize("cfg,T", [(C2, 3), (C5, 4), (C2, 10)])
def test_masked_forward_through_slots_ignores_workspace_contents(cfg, T):
    print(f"workspace garbage masked+slots {cfg.name} T={T}", flush=True)
    ld = LayerData(cfg, 1, 6, T)
    mask = np.array([0x5A5A5A5A, 0xF0F0F0F0, 0x0FF00FF0, 0x33CC33CC, 0xAAAA5555, 0x1, 0xFFFF, 0x80000000],
                    dtype=np.uint32)[:(cfg.n_experts + 31) // 32]
    a = run(ld, 0, mask=mask, slots=True)
    b = run(ld, 0xFF, mask=mask, slots=True)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


@pytest.mark.parametrize("T", [1, 4])
def test_fused_route_forward_ignores_workspace_contents(T):
    """ft_moe_route_forward on the bf16 decode layer: selection inside the
    gate/up kernel at one token, the two-call branch at four."""
    print(f"workspace garbage fused C2 T={T}", flush=True)
    cfg = C2
    ld = LayerData(cfg, 2, 8, T)
    r_ids, _, _ = ld.gpu_route()
    ld.build_pool(r_ids.cpu().numpy().ravel())   # the selected records; every other one is poison
    res = []
    for fill in (0, 0xFF):
        ws = torch.full((ftmoe.ft_moe_route_forward_workspace_bytes(ld.desc, T),), fill, dtype=torch.uint8,
                        device="cuda")
        ids = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
        gates = torch.empty((T, cfg.top_k), dtype=torch.float32, device="cuda")
        out = torch.empty((T, cfg.hidden), dtype=torch.float32, device="cuda")
        ftmoe.ft_moe_route_forward(ld.desc, dev(ld.x), dev(ld.wr), ids, gates, ld.pool, out, ws)
        torch.cuda.synchronize()
        res.append((ids, gates, out))
    for x, y in zip(*res):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    assert not torch.isnan(res[0][2]).any()
