"""GPU: the decode configuration the benchmark times, checked as it is timed.

The benchmark captures the fused ft_moe_route_forward calls of consecutive
layers of the 2048/768/128-expert/top-8 bf16 layer into one HIP graph on a
side stream and replays it.  Here three such layers at 1, 2 and 4 tokens are
captured the same way; every replay (three, with eager work and
synchronisations in between) must give, bit for bit, the ids, gates and
outputs of the same calls launched eagerly, and those must match the oracle:
ids exactly, gates to 1e-6, outputs within 1e-2 max relative error.  Each
layer's pool holds real records only for the experts the oracle selects;
every other record is NaN bytes, so a wrong selection cannot pass."""
import numpy as np
import pytest
import torch

from gpu_util import LayerData, dev, max_rel_err
from sparse_moe_expert_softmax_amd import ftmoe
from sparse_moe_expert_softmax_amd.configs import C2

pytestmark = pytest.mark.gpu

N_LAYERS = 3


@pytest.mark.parametrize("T", [1, 2, 4])
def test_graph_replayed_fused_decode_layers_match_eager_and_oracle(T):
    print(f"graph-captured fused C2 decode, {N_LAYERS} layers, T={T}", flush=True)
    cfg, k, H = C2, C2.top_k, C2.hidden
    lds = [LayerData(cfg, layer, 700 + T, T) for layer in range(N_LAYERS)]
    refs = []
    for ld in lds:
        ref, o_ids, o_gates = ld.oracle_layer()
        ld.build_pool(o_ids.ravel())
        refs.append((ref, o_ids, o_gates))
    xs = [dev(ld.x) for ld in lds]
    wrs = [dev(ld.wr) for ld in lds]
    ws = torch.zeros(ftmoe.ft_moe_route_forward_workspace_bytes(lds[0].desc, T), dtype=torch.uint8, device="cuda")

    def buffers():
        return ([torch.full((T, k), -7, dtype=torch.int32, device="cuda") for _ in lds],
                [torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda") for _ in lds],
                [torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda") for _ in lds])

    def layers(ids, gates, outs, st):
        for i, ld in enumerate(lds):
            ftmoe.ft_moe_route_forward(ld.desc, xs[i], wrs[i], ids[i], gates[i], ld.pool, outs[i], ws, stream=st)

    e_ids, e_gates, e_out = buffers()
    layers(e_ids, e_gates, e_out, torch.cuda.current_stream())
    torch.cuda.synchronize()
    for i, (ref, o_ids, o_gates) in enumerate(refs):
        assert np.array_equal(e_ids[i].cpu().numpy(), o_ids), f"layer {i}: ids differ from the oracle"
        assert np.max(np.abs(e_gates[i].cpu().numpy() - o_gates)) <= 1e-6
        err = max_rel_err(e_out[i].cpu().numpy(), ref)
        assert err <= 1e-2, f"layer {i}: max relative error {err:.3g}"

    g_ids, g_gates, g_out = buffers()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            layers(g_ids, g_gates, g_out, torch.cuda.current_stream())
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in g_ids + g_gates + g_out:
            t.fill_(-1)  # the replay must rewrite every output
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i in range(N_LAYERS):
            assert torch.equal(g_ids[i], e_ids[i]), f"replay {rep}, layer {i}: ids"
            assert torch.equal(g_gates[i].view(torch.int32), e_gates[i].view(torch.int32)), f"replay {rep}, layer {i}: gates"
            assert torch.equal(g_out[i].view(torch.int32), e_out[i].view(torch.int32)), f"replay {rep}, layer {i}: out"
        # eager work between replays, on the same workspace
        layers(e_ids, e_gates, e_out, torch.cuda.current_stream())
        torch.cuda.synchronize()
