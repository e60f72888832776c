"""Host-side argument checks of the graph-capturable decode step (no GPU:
every check runs before any device memory is touched)."""
import pytest
import torch

from sparse_moe_expert_softmax_amd import ftmoe, synth
from sparse_moe_expert_softmax_amd.configs import BF16, MXFP4, MoEConfig
from sparse_moe_expert_softmax_amd.decode_step import DeviceFetchStep

CFG = MoEConfig("step_args_mxfp4", 85, hidden=512, inter=256, n_experts=16, top_k=2, act_dtype=BF16,
                router_dtype=BF16, w_dtype=MXFP4, n_layers=2)


def _args(n_slots=6, pool_rows=6, table_bytes=None, n_routers=2):
    stride = synth.record_stride(CFG.hidden, CFG.inter, CFG.w_dtype)
    desc = ftmoe.make_desc(CFG, stride)
    tb = ftmoe.ft_slot_table_bytes(CFG.n_layers, CFG.n_experts, n_slots) if table_bytes is None else table_bytes
    table = torch.zeros(tb, dtype=torch.uint8)
    pool = torch.zeros((pool_rows, stride), dtype=torch.uint8)
    routers = [torch.zeros(1)] * n_routers
    srcs = [torch.zeros(CFG.n_experts, dtype=torch.int64)] * 2
    return desc, table, pool, routers, srcs, n_slots


@pytest.mark.parametrize("kw,msg", [({"pool_rows": 5}, "pool must hold"), ({"table_bytes": 64}, "slot table"),
                                    ({"n_routers": 1}, "one router")])
def test_decode_step_rejects_mismatched_buffers(kw, msg):
    desc, table, pool, routers, srcs, S = _args(**kw)
    rb = synth.record_bytes(CFG.hidden, CFG.inter, CFG.w_dtype)
    with pytest.raises(ValueError, match=msg):
        DeviceFetchStep(desc, CFG.n_layers, 1, table, S, pool, rb, routers, srcs)
