"""GPU: the allocation-free route + forward (ft_moe_route_forward_noalloc)
against ft_moe_route_forward with a caller workspace, on the same inputs.

Bar: ids, gates and outputs bitwise equal (the same kernels run on the same
inputs; only the workspace address differs).  Calls follow one another on
the library's one scratch array, the second smaller than the first, so a
call must not depend on what the previous one left there."""
import numpy as np
import pytest
import torch

from gpu_util import LayerData, dev
from sparse_moe_expert_softmax_amd import ftmoe
from sparse_moe_expert_softmax_amd.configs import C1, C2, C3, C4, C5

pytestmark = pytest.mark.gpu


def both(cfg, T, step, bias=None, mask=None):
    ld = LayerData(cfg, 0, step, T)
    ids_r, _, _ = ld.gpu_route(bias=bias)
    ld.build_pool(ids_r.cpu().numpy().ravel())
    k, H = cfg.top_k, cfg.hidden
    b = None if bias is None else dev(bias.astype(np.float32))
    m = None if mask is None else dev(np.asarray(mask, dtype=np.uint32))
    res = []
    for noalloc in (False, True):
        ids = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
        gates = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
        out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            ftmoe.ft_moe_route_forward_noalloc(ld.desc, dev(ld.x), dev(ld.wr), ids, gates, ld.pool, out,
                                               sel_bias=b, expert_mask=m)
        else:
            ws = torch.empty(ftmoe.ft_moe_route_forward_workspace_bytes(ld.desc, T), dtype=torch.uint8,
                             device="cuda")
            ftmoe.ft_moe_route_forward(ld.desc, dev(ld.x), dev(ld.wr), ids, gates, ld.pool, out, ws,
                                       sel_bias=b, expert_mask=m)
        torch.cuda.synchronize()
        res.append((ids, gates, out))
    (i0, g0, o0), (i1, g1, o1) = res
    assert torch.equal(i0, i1)
    assert torch.equal(g0.view(torch.int32), g1.view(torch.int32))
    assert torch.equal(o0.view(torch.int32), o1.view(torch.int32))
    assert not torch.isnan(o1).any()


@pytest.mark.parametrize("cfg,first,second", [(C2, 4, 1), (C3, 3, 1), (C1, 16, 5)])
def test_noalloc_matches_workspace_call_twice_in_a_row(cfg, first, second):
    """bf16 decode: 4 tokens (selection as its own launch) then 1 (selection
    inside the gate/up kernel); MXFP4 with a selection bias; the fp32 layer."""
    print(f"noalloc {cfg.name} T={first} then T={second}", flush=True)
    g = np.random.default_rng(first * 10 + second)
    for T in (first, second):
        bias = g.normal(0.0, 0.5, (T, cfg.n_experts)) if cfg is C3 else None
        both(cfg, T, 200 + T, bias=bias)


def test_noalloc_with_partition_mask():
    print("noalloc C5 T=4 masked, then T=2", flush=True)
    m = np.array([0xA5A5A5A5, 0x0F0F0F0F, 0xFFFF0000, 0x12345678, 0x0, 0xFFFFFFFF, 0x3C3C3C3C, 0x55555555],
                 dtype=np.uint32)
    both(C5, 4, 210, mask=m)
    both(C5, 2, 211, mask=m)


def test_noalloc_rejects_calls_beyond_its_scratch_before_any_launch():
    cfg, T = C4, 8192
    desc = ftmoe.make_desc(cfg)
    assert ftmoe.ft_moe_route_forward_workspace_bytes(desc, T) > ftmoe.FT_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, cfg.hidden), dtype=torch.int16, device="cuda")
    wr = torch.zeros((cfg.n_experts, cfg.hidden), dtype=torch.int16, device="cuda")
    ids = torch.zeros((T, cfg.top_k), dtype=torch.int32, device="cuda")
    gates = torch.zeros((T, cfg.top_k), dtype=torch.float32, device="cuda")
    out = torch.zeros((T, cfg.hidden), dtype=torch.float32, device="cuda")
    pool = torch.zeros(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(ftmoe.FtError) as ei:
        ftmoe.ft_moe_route_forward_noalloc(desc, x, wr, ids, gates, pool, out)
    assert ei.value.status == ftmoe.FT_EWORKSPACE
    assert "allocation-free" in str(ei.value)
    torch.cuda.synchronize()
    assert not ids.any() and not out.any()
