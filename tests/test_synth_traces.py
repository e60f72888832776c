"""CPU checks of the synthetic expert traces the LRU workload and the
placement study use: seeded (the same call gives the same trace), ids in
range, k distinct experts per token, and for the trace with temporal
locality a kept fraction near the requested probability."""
import numpy as np

from sparse_moe_expert_softmax_amd import synth
from sparse_moe_expert_softmax_amd.configs import C3


def _valid(tr):
    assert tr.min() >= 0 and tr.max() < C3.n_experts
    flat = tr.reshape(-1, C3.top_k)
    assert all(len(set(r)) == C3.top_k for r in flat)


def test_zipf_trace_seeded_and_valid():
    a = synth.zipf_trace(C3, n_steps=64, n_tokens=2)
    assert a.shape == (64, C3.n_layers, 2, C3.top_k)
    assert np.array_equal(a, synth.zipf_trace(C3, n_steps=64, n_tokens=2))
    _valid(a)


def test_sticky_trace_keeps_about_p_of_the_experts():
    p = 0.8
    a = synth.sticky_trace(C3, 200, 2, p)
    assert a.shape == (200, C3.n_layers, 2, C3.top_k)
    assert np.array_equal(a, synth.sticky_trace(C3, 200, 2, p))
    _valid(a)
    kept = np.mean([len(set(a[s, l, t]) & set(a[s + 1, l, t])) / C3.top_k
                    for s in range(199) for l in range(0, C3.n_layers, 7) for t in range(2)])
    # kept with probability p, plus a redrawn expert that happens to repeat
    assert p - 0.03 < kept < p + 0.08
    # p = 0 keeps only what the popularity law redraws by chance
    b = synth.sticky_trace(C3, 50, 1, 0.0)
    kept0 = np.mean([len(set(b[s, 0, 0]) & set(b[s + 1, 0, 0])) / C3.top_k for s in range(49)])
    assert kept0 < 0.5


def test_layer_correlated_activations_have_the_stated_correlation():
    from sparse_moe_expert_softmax_amd import synth
    from sparse_moe_expert_softmax_amd.configs import C3
    from oracle.formats import bf16_bits_to_f64
    for alpha in (0.0, 0.9):
        x = bf16_bits_to_f64(synth.layer_correlated_activations(C3, 0, 4, alpha))   # [43, 4, 4096]
        a, b = x[:-1].ravel(), x[1:].ravel()
        assert abs(np.corrcoef(a, b)[0, 1] - alpha) < 0.01
        assert abs(x.std() - 1.0) < 0.01
    same = synth.layer_correlated_activations(C3, 3, 2, 0.9)
    assert np.array_equal(same, synth.layer_correlated_activations(C3, 3, 2, 0.9))
