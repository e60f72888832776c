"""GPU: a whole decode step with device-side miss handling (route, slot
lookup, fetch from pinned host memory, forward, for every layer), captured
once as a HIP graph and replayed step after step.

Each replay is checked against the oracle (ids bit-exact and gates within
1e-6 under the step's selection bias; slots, miss flags and miss lists
bit-exact against the LRU state machine; outputs within 1e-2 relative error
of the fp64 layer) and bit for bit against the same sequence launched
eagerly on a second table and pool.  Between replays the test does its own
eager work and synchronises, so that a graph that only works once, or that
keeps state from its capture, fails."""
import numpy as np
import pytest
import torch

from gpu_util import LayerData, dev, max_rel_err
from oracle.lru import LruSim
from sparse_moe_expert_softmax_amd import ftmoe, synth
from sparse_moe_expert_softmax_amd.configs import BF16, MXFP4, MoEConfig
from sparse_moe_expert_softmax_amd.decode_step import DeviceFetchStep

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

CFG = MoEConfig("graph_mxfp4_h512_i256", 98, hidden=512, inter=256, n_experts=32, top_k=4, act_dtype=BF16,
                router_dtype=BF16, w_dtype=MXFP4, n_layers=3)


def _make(cfg, S, T, host, routers):
    L, E = cfg.n_layers, cfg.n_experts
    stride = synth.record_stride(cfg.hidden, cfg.inter, cfg.w_dtype)
    rb = synth.record_bytes(cfg.hidden, cfg.inter, cfg.w_dtype)
    table = torch.zeros(ftmoe.ft_slot_table_bytes(L, E, S), dtype=torch.uint8, device="cuda")
    ftmoe.ft_slot_table_init(table, L, E, S)
    pool = torch.full((S, stride), 0xFF, dtype=torch.uint8, device="cuda")
    src = [torch.tensor([h.data_ptr() for h in host[l]], dtype=torch.int64, device="cuda") for l in range(L)]
    return DeviceFetchStep(ftmoe.make_desc(cfg, stride), L, T, table, S, pool, rb, routers, src)


def _stage(st, xs, biases):
    for l in range(st.L):
        st.x[l].view(torch.int16).copy_(dev(xs[l]))
        st.bias[l].copy_(torch.from_numpy(biases[l].astype(np.float32)))


@pytest.mark.parametrize("T,S", [(1, 20), (3, 24)])
def test_graph_replayed_decode_step_matches_oracle_and_eager(T, S):
    cfg = CFG
    L, E, k = cfg.n_layers, cfg.n_experts, cfg.top_k
    print(f"graph decode step T={T} S={S}", flush=True)
    recs = [[synth.expert_record(cfg, l, e) for e in range(E)] for l in range(L)]
    host = [[torch.from_numpy(r).pin_memory() for r in recs[l]] for l in range(L)]
    routers = [dev(synth.router_weights(cfg, l)) for l in range(L)]
    g_step = _make(cfg, S, T, host, routers)
    e_step = _make(cfg, S, T, host, routers)
    g_step.capture()
    torch.cuda.synchronize()
    # capture launched nothing: the graph's table is still the initial one
    assert torch.equal(g_step.table, e_step.table)
    sim = LruSim(L, E, S)
    rng = np.random.default_rng(2026 + T)
    hot = [rng.choice(E, 10, replace=False) for _ in range(L)]  # a popular subset per layer
    n_miss_total = n_hit_total = 0
    for step in range(6):
        xs = [synth.activations(cfg, step, l, T) for l in range(L)]
        biases = []
        for l in range(L):
            b = np.zeros((T, E))
            for t in range(T):
                pick = hot[l] if rng.random() < 0.8 else np.arange(E)
                b[t, rng.choice(pick, k, replace=False)] = 30.0
            biases.append(b)
        _stage(g_step, xs, biases)
        _stage(e_step, xs, biases)
        g_step.run()
        e_step.enqueue()
        torch.cuda.synchronize()
        for name in ("ids", "gates", "slots", "flags", "out"):
            a, b = getattr(g_step, name), getattr(e_step, name)
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (step, name)
        for l in range(L):
            nm = int(g_step.mlist[l, 0])
            assert nm == int(e_step.mlist[l, 0])
            assert torch.equal(g_step.mlist[l, 1:1 + 2 * nm], e_step.mlist[l, 1:1 + 2 * nm])
        assert torch.equal(g_step.table, e_step.table) and torch.equal(g_step.pool, e_step.pool)
        # against the oracle
        for l in range(L):
            ld = LayerData(cfg, l, step, T, x=xs[l])
            o_ids, o_gates, _ = ld.oracle_route(biases[l])
            np.testing.assert_array_equal(g_step.ids[l].cpu().numpy(), o_ids)
            np.testing.assert_allclose(g_step.gates[l].cpu().numpy(), o_gates, rtol=0, atol=1e-6)
            ref = sim.lookup(l, o_ids)
            assert ref is not None
            np.testing.assert_array_equal(g_step.slots[l].cpu().numpy().ravel(), np.ravel(ref[0]))
            np.testing.assert_array_equal(g_step.flags[l].cpu().numpy().ravel(), np.ravel(ref[1]))
            ml = g_step.mlist[l].cpu().numpy()
            assert ml[0] == len(ref[2])
            assert [tuple(ml[1 + 2 * i:3 + 2 * i]) for i in range(ml[0])] == [tuple(p) for p in ref[2]]
            n_miss_total += int(ml[0])
            n_hit_total += len(set(o_ids.ravel().tolist())) - int(ml[0])
            o_out, _, _ = ld.oracle_layer(bias=biases[l])
            out = g_step.out[l].cpu().numpy()
            assert not np.isnan(out).any()
            assert max_rel_err(out, o_out) <= 1e-2, (step, l)
        # eager work of the test's own between replays
        e_step.out.fill_(float("nan"))
        torch.cuda.synchronize()
    assert n_miss_total > 0 and n_hit_total > 0  # both paths of the lookup were taken
