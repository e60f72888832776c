"""Expert placement policies at equal capacity (the library's global LRU, a
per-layer LRU split, a profiled static set): miss counts per (step, layer).

CPU: the profiled static set against a direct recount.  GPU: both LRU
policies, run on the slot-table kernel, against the LRU state machine of
the oracle, call by call."""
import numpy as np
import pytest

from oracle.lru import LruSim
from sparse_moe_expert_softmax_amd import placement, synth
from sparse_moe_expert_softmax_amd.configs import C3


def test_profiled_static_set_counts_misses_of_unprofiled_keys():
    g = np.random.default_rng(5)
    steps, L, n, E, S, prof = 40, 3, 4, 10, 7, 8
    tr = g.integers(0, E, size=(steps, L, n))
    got = placement.profiled_static_misses(tr, E, S, prof)
    # direct recount: how often each key was selected in the profiled steps
    counts = {}
    for s in range(prof):
        for l in range(L):
            for e in set(tr[s, l].tolist()):
                counts[(l, e)] = counts.get((l, e), 0) + 1
    keys = sorted(counts, key=lambda key: (-counts[key], key[0] * E + key[1]))[:S]
    resident = set(keys)
    for s in range(steps):
        for l in range(L):
            want = sum(1 for e in set(tr[s, l].tolist()) if (l, e) not in resident)
            assert got[s, l] == want
    assert placement.distinct_selected(tr)[3, 1] == len(set(tr[3, 1].tolist()))


@pytest.mark.gpu
@pytest.mark.parametrize("b", [1, 4])
def test_lru_policies_match_the_state_machine(b):
    """300 steps of the Zipf(1.1) trace of the 284B-like layer (43 layers,
    256 experts, 2,752 slots): global LRU and the per-layer split (64 slots
    per layer) against LruSim, every call."""
    import torch
    cfg = C3
    L, E, S, k = cfg.n_layers, cfg.n_experts, cfg.n_slots, cfg.top_k
    tr = synth.zipf_trace(cfg, n_steps=300)[:, :, :b, :].reshape(300, L, b * k)
    print(f"placement b={b}", flush=True)
    g = placement.lru_misses(torch, tr, E, S, per_layer=False)
    p = placement.lru_misses(torch, tr, E, S, per_layer=True)
    sim_g = LruSim(L, E, S)
    sim_p = [LruSim(1, E, S // L) for _ in range(L)]
    for s in range(300):
        for l in range(L):
            assert g[s, l] == len(sim_g.lookup(l, tr[s, l])[2])
            assert p[s, l] == len(sim_p[l].lookup(0, tr[s, l])[2])
    assert g.sum() > 0 and p.sum() > 0
