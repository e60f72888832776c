"""GPU: workspaces need no initialisation.  Route and forward run once with
zero-filled workspaces and once with workspaces full of 0xFF bytes (NaN in
every float view, -1 in every integer view); ids, gates and outputs must be
bitwise equal.  Covers the decode route and GEMV path, the general path,
the many-token bounded router and the prefill MFMA path."""
import numpy as np
import pytest
import torch

from gpu_util import LayerData, dev
from sparse_moe_expert_softmax_amd import ftmoe
from sparse_moe_expert_softmax_amd.configs import BF16, C2, C3, MXFP4, MoEConfig

pytestmark = pytest.mark.gpu

MID = MoEConfig("prefill_mid_mxfp4", 91, hidden=512, inter=384, n_experts=16, top_k=4, act_dtype=BF16,
                router_dtype=BF16, w_dtype=MXFP4, n_layers=1)


def run(ld, fill):
    cfg, T = ld.cfg, ld.T
    rws = torch.full((max(ftmoe.ft_route_workspace_bytes(ld.desc, T), 256),), fill, dtype=torch.uint8, device="cuda")
    fws = torch.full((max(ftmoe.ft_moe_workspace_bytes(ld.desc, T), 256),), fill, dtype=torch.uint8, device="cuda")
    ids = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, cfg.top_k), dtype=torch.float32, device="cuda")
    ftmoe.ft_moe_route(ld.desc, dev(ld.x), dev(ld.wr), ids, gates, workspace=rws)
    torch.cuda.synchronize()
    ld.build_pool(ids.cpu().numpy().ravel())
    out = torch.empty((T, cfg.hidden), dtype=torch.float32, device="cuda")
    ftmoe.ft_moe_forward(ld.desc, dev(ld.x), ids, gates, ld.pool, out, fws)
    torch.cuda.synchronize()
    return ids, gates, out


@pytest.mark.parametrize("cfg,T", [(C2, 1), (C2, 4), (C2, 17), (C3, 2), (MID, 300)])
def test_results_do_not_depend_on_workspace_contents(cfg, T):
    print(f"workspace garbage {cfg.name} T={T}", flush=True)
    ld = LayerData(cfg, 0, 3, T)
    a = run(ld, 0)
    b = run(ld, 0xFF)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    assert not torch.isnan(a[2]).any()
