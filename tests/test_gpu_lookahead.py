"""GPU: decode with look-ahead prefetch (LookaheadStep): at every layer, the
next layer's router on this layer's input predicts its experts, which are
looked up and copied into the cache on a side stream while this layer
computes.

Each replay of the captured step is checked against the oracle and the LRU
state machine, and bit for bit against the same sequence launched eagerly:
ids and gates bit-exact / within 1e-6 (real and predicted), slots, miss
flags and miss lists of both lookups per layer bit-exact against LruSim fed
(real ids of layer l, predicted ids of layer l+1) in order, outputs within
1e-2 of the fp64 layer (so every record the forward reads had landed).
Inputs drift from layer to layer (correlation 0.95), so predictions hit."""
import numpy as np
import pytest
import torch

from gpu_util import LayerData, dev, max_rel_err
from oracle.lru import LruSim
from oracle.moe import route, to_f64
from sparse_moe_expert_softmax_amd import ftmoe, synth
from sparse_moe_expert_softmax_amd.configs import BF16, MXFP4, MoEConfig
from sparse_moe_expert_softmax_amd.lookahead import LookaheadStep

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

CFG = MoEConfig("lookahead_mxfp4_h512_i256", 125, hidden=512, inter=256, n_experts=32, top_k=4, act_dtype=BF16,
                router_dtype=BF16, w_dtype=MXFP4, n_layers=4)


def _make(cfg, S, T, host, routers):
    L, E = cfg.n_layers, cfg.n_experts
    stride = synth.record_stride(cfg.hidden, cfg.inter, cfg.w_dtype)
    rb = synth.record_bytes(cfg.hidden, cfg.inter, cfg.w_dtype)
    table = torch.zeros(ftmoe.ft_slot_table_bytes(L, E, S), dtype=torch.uint8, device="cuda")
    ftmoe.ft_slot_table_init(table, L, E, S)
    pool = torch.full((S, stride), 0xFF, dtype=torch.uint8, device="cuda")
    src = [torch.tensor([h.data_ptr() for h in host[l]], dtype=torch.int64, device="cuda") for l in range(L)]
    return LookaheadStep(ftmoe.make_desc(cfg, stride), L, T, table, S, pool, rb, routers, src)


def _check_lookup(sim, layer, ids, slots, flags, mlist):
    ref = sim.lookup(layer, ids)
    assert ref is not None
    np.testing.assert_array_equal(slots.ravel(), np.ravel(ref[0]))
    np.testing.assert_array_equal(flags.ravel(), np.ravel(ref[1]))
    assert mlist[0] == len(ref[2])
    assert [tuple(mlist[1 + 2 * i:3 + 2 * i]) for i in range(mlist[0])] == [tuple(p) for p in ref[2]]
    return len(ref[2])


@pytest.mark.parametrize("T,S", [(1, 20), (2, 28)])
def test_lookahead_step_matches_oracle_lru_and_eager(T, S):
    cfg = CFG
    L, E = cfg.n_layers, cfg.n_experts
    print(f"lookahead step T={T} S={S}", flush=True)
    host = [[torch.from_numpy(synth.expert_record(cfg, l, e)).pin_memory() for e in range(E)] for l in range(L)]
    routers = [dev(synth.router_weights(cfg, l)) for l in range(L)]
    g_step = _make(cfg, S, T, host, routers)
    e_step = _make(cfg, S, T, host, routers)
    g_step.capture()
    torch.cuda.synchronize()
    assert torch.equal(g_step.table, e_step.table)
    sim = LruSim(L, E, S)
    w64 = [to_f64(synth.router_weights(cfg, l), cfg.router_dtype) for l in range(L)]
    hits = total = 0
    for step in range(5):
        xs = synth.layer_correlated_activations(cfg, step, T, 0.95)
        for st in (g_step, e_step):
            st.x.view(torch.int16).copy_(dev(xs))
        g_step.run()
        e_step.enqueue()
        torch.cuda.synchronize()
        for name in ("ids", "gates", "slots", "flags", "out"):
            a, b = getattr(g_step, name), getattr(e_step, name)
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (step, name)
        for l in range(L):  # miss lists: the count and the entries it covers
            nm = int(g_step.mlist[l, 0])
            assert nm == int(e_step.mlist[l, 0])
            assert torch.equal(g_step.mlist[l, 1:1 + 2 * nm], e_step.mlist[l, 1:1 + 2 * nm])
        assert torch.equal(g_step.pred_ids[1:], e_step.pred_ids[1:]) and torch.equal(g_step.table, e_step.table)
        assert torch.equal(g_step.pool, e_step.pool)
        ids = g_step.ids.cpu().numpy()
        pred = g_step.pred_ids.cpu().numpy()
        for l in range(L):
            ld = LayerData(cfg, l, step, T, x=xs[l])
            o_ids, o_gates, _ = ld.oracle_route()
            np.testing.assert_array_equal(ids[l], o_ids)
            np.testing.assert_allclose(g_step.gates[l].cpu().numpy(), o_gates, rtol=0, atol=1e-6)
            _check_lookup(sim, l, o_ids, g_step.slots[l].cpu().numpy(), g_step.flags[l].cpu().numpy(),
                          g_step.mlist[l].cpu().numpy())
            if l + 1 < L:  # the prediction: layer l+1's router on x_l
                p_ids, _, _ = route(to_f64(xs[l], cfg.act_dtype), w64[l + 1], cfg.top_k)
                np.testing.assert_array_equal(pred[l + 1], p_ids)
                _check_lookup(sim, l + 1, p_ids, g_step.pslots[l + 1].cpu().numpy(),
                              g_step.pflags[l + 1].cpu().numpy(), g_step.pmlist[l + 1].cpu().numpy())
            if l >= 1:
                hits += len(set(pred[l].ravel()) & set(ids[l].ravel()))
                total += len(set(ids[l].ravel()))
            o_out, _, _ = ld.oracle_layer()
            out = g_step.out[l].cpu().numpy()
            assert not np.isnan(out).any()
            assert max_rel_err(out, o_out) <= 1e-2, (step, l)
        e_step.out.fill_(float("nan"))
        torch.cuda.synchronize()
    print(f"  predicted experts used: {hits} of {total}", flush=True)
    assert hits > total // 4
