"""GPU: the double-buffered prefill pipeline (ft_prefill_pipeline_start /
_layer).  Every layer is computed from the device buffer that its own copy
filled while the previous layer ran; each layer's ids, gates and outputs are
checked against the oracle, and a corrupted host record must change exactly
the outputs of the layer it belongs to (negative control: the computed layer
really is the uploaded one)."""
import numpy as np
import pytest
import torch

from gpu_util import LayerData, dev, max_rel_err
from oracle.mx import bf16_round_f32, mxfp8_two_term, mxfp8_two_term_f32
from sparse_moe_expert_softmax_amd import ftmoe, synth
from sparse_moe_expert_softmax_amd.configs import BF16, MXFP4, NVFP4, MoEConfig
from sparse_moe_expert_softmax_amd.prefill_pipeline import PrefillPipeline

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

PIPE_MX = MoEConfig("pipeline_mxfp4", 95, hidden=256, inter=256, n_experts=8, top_k=2, act_dtype=BF16,
                    router_dtype=BF16, w_dtype=MXFP4, n_layers=5)
PIPE_BF16 = MoEConfig("pipeline_bf16", 96, hidden=512, inter=256, n_experts=16, top_k=4, act_dtype=BF16,
                      router_dtype=BF16, w_dtype=BF16, n_layers=4)
PIPE_NV = MoEConfig("pipeline_nvfp4", 138, hidden=512, inter=256, n_experts=16, top_k=4, act_dtype=BF16,
                    router_dtype=BF16, w_dtype=NVFP4, n_layers=3)


def _host_layers(cfg):
    """Pinned host records [E, stride] per layer (host generator)."""
    return [torch.from_numpy(synth.layer_records(cfg, l)).pin_memory() for l in range(cfg.n_layers)]


def _run(cfg, T, host, lds):
    L, k, H = cfg.n_layers, cfg.top_k, cfg.hidden
    desc = lds[0].desc
    rec = synth.record_bytes(cfg.hidden, cfg.inter, cfg.w_dtype)
    pp = PrefillPipeline(desc, rec)
    ptrs = [[host[l][e].data_ptr() for e in range(cfg.n_experts)] for l in range(L)]
    ids = torch.full((L, T, k), -1, dtype=torch.int32, device="cuda")
    gates = torch.full((L, T, k), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((L, T, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(ftmoe.ft_moe_route_forward_workspace_bytes(desc, T), dtype=torch.uint8, device="cuda")
    xs = [dev(ld.x) for ld in lds]
    wrs = [dev(ld.wr) for ld in lds]
    pp.start(ptrs[0])
    for l in range(L):
        pp.layer(ptrs[l + 1] if l + 1 < L else None, xs[l], wrs[l], ids[l], gates[l], out[l], ws)
    torch.cuda.synchronize()
    assert pp.n_done == L
    with pytest.raises(ftmoe.FtError) as ei:     # no layer L was ever uploaded
        pp.layer(None, xs[0], wrs[0], ids[0], gates[0], out[0], ws)
    assert ei.value.status == ftmoe.FT_EINVAL
    return ids.cpu().numpy(), gates.cpu().numpy(), out.cpu().numpy()


@pytest.mark.parametrize("cfg,T", [(PIPE_MX, 300), (PIPE_BF16, 3), (PIPE_BF16, 300), (PIPE_NV, 300)])
def test_pipeline_layers_match_oracle_and_a_corrupted_record_shows(cfg, T):
    """MXFP4 at 300 tokens (scaled matrix cores, five layers), bf16 at 3
    tokens (decode path with in-kernel selection, four layers), bf16 and
    NVFP4 at 300 tokens (bf16 matrix cores)."""
    print(f"prefill pipeline {cfg.name} T={T} layers={cfg.n_layers}", flush=True)
    host = _host_layers(cfg)
    lds = [LayerData(cfg, l, 7 + l, T) for l in range(cfg.n_layers)]
    ids, gates, out = _run(cfg, T, host, lds)
    mx = cfg.w_dtype == MXFP4
    for l, ld in enumerate(lds):
        ld._records = {e: host[l][e].numpy() for e in range(cfg.n_experts)}
        q = dict(x_quant=mxfp8_two_term, h_quant=mxfp8_two_term_f32, y_quant=bf16_round_f32) if mx else {}
        ref, o_ids, o_gates = ld.oracle_layer(**q)
        np.testing.assert_array_equal(ids[l], o_ids)
        np.testing.assert_allclose(gates[l], o_gates, rtol=0, atol=1e-6)
        err = max_rel_err(out[l], ref)
        assert err <= 1e-2, f"layer {l}: max rel err {err:.3g}"
    # negative control: flip one routed expert record of layer 2 on the host
    victim = int(ids[2, 0, 0])
    rec = synth.record_bytes(cfg.hidden, cfg.inter, cfg.w_dtype)
    host[2][victim, : rec // 2] = host[2][victim, rec // 2 : 2 * (rec // 2)].clone()
    ids2, gates2, out2 = _run(cfg, T, host, lds)
    for l in range(cfg.n_layers):
        np.testing.assert_array_equal(ids2[l], ids[l])
        if l == 2:
            assert not np.array_equal(out2[l], out[l])
        else:
            assert np.array_equal(out2[l], out[l])
