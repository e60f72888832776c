"""GPU: the many-token router without a logits output (bf16 x and W_r,
renormalized gates) against the fp64 oracle.

That path picks candidates from bf16 matrix-core scores with a rounding
bound and recomputes only the candidates exactly, so the cases aim at the
bound: real prefill shapes, ragged token / expert / hidden sizes (and rows
longer than the 4096 elements the exact pass keeps in registers), experts
whose scores differ by far less than the bound (and exact duplicates, where
the lowest id must win), rows whose norms overflow fp32 (every expert is
recomputed) or whose products fall below fp32's normal range (the bound's
absolute term makes every expert a candidate), and a selection bias.

Bars: ids bit-exact; gates within 1e-6 of the oracle; ids and gates equal to
those of the full fp64 path (ft_moe_route with a logits output)."""
import numpy as np
import pytest
import torch

from gpu_util import LayerData, dev
from sparse_moe_expert_softmax_amd import ftmoe, synth
from sparse_moe_expert_softmax_amd.configs import BF16, C2, C3, C4, C5, MoEConfig

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

RAGGED = MoEConfig("router_e40_h384", 95, hidden=384, inter=128, n_experts=40, top_k=3, act_dtype=BF16,
                   router_dtype=BF16, w_dtype=BF16, n_layers=1)
WIDE = MoEConfig("router_e1000_h512", 96, hidden=512, inter=128, n_experts=1000, top_k=4, act_dtype=BF16,
                 router_dtype=BF16, w_dtype=BF16, n_layers=1)


def route_bounded(ld: LayerData, bias=None):
    cfg, T = ld.cfg, ld.T
    ids = torch.full((T, cfg.top_k), -7, dtype=torch.int32, device="cuda")
    gates = torch.full((T, cfg.top_k), float("nan"), dtype=torch.float32, device="cuda")
    b = None if bias is None else dev(bias.astype(np.float32))
    ws = torch.zeros(ftmoe.ft_route_workspace_bytes(ld.desc, T), dtype=torch.uint8, device="cuda")
    ftmoe.ft_moe_route(ld.desc, dev(ld.x), dev(ld.wr), ids, gates, sel_bias=b, logits=None, workspace=ws)
    torch.cuda.synchronize()
    return ids, gates


def check(ld: LayerData, bias=None):
    assert ld.T > 16 and ld.cfg.renormalize
    ids, gates = route_bounded(ld, bias)
    o_ids, o_gates, _ = ld.oracle_route(bias)
    np.testing.assert_array_equal(ids.cpu().numpy(), o_ids)
    np.testing.assert_allclose(gates.cpu().numpy(), o_gates, rtol=0, atol=1e-6)
    f_ids, f_gates, _ = ld.gpu_route(bias)  # fp64 logits of every expert
    torch.cuda.synchronize()
    assert torch.equal(ids, f_ids)
    np.testing.assert_allclose(gates.cpu().numpy(), f_gates.cpu().numpy(), rtol=0, atol=1e-7)
    return ids


@pytest.mark.parametrize("cfg,T", [(C4, 300), (C2, 17), (C2, 1031), (RAGGED, 65), (WIDE, 70), (C5, 70)])
def test_bounded_router_matches_oracle(cfg, T):
    print(f"bounded route {cfg.name} T={T}", flush=True)
    check(LayerData(cfg, 0, 5, T))


def test_bounded_router_near_ties_and_duplicates():
    """32 groups of 8 experts: each row is its group's base row with one
    element moved by one bf16 step, so scores within a group differ by
    ~1e-4 while the bound is ~4e-2; the last two rows of every group repeat
    the group's first row exactly."""
    cfg = C4
    base = synth.router_weights(cfg, 2).view(np.uint16).reshape(cfg.n_experts, cfg.hidden)
    r = np.random.default_rng(11)
    wr = np.empty_like(base)
    for grp in range(32):
        b = base[8 * grp]
        for j in range(8):
            row = b.copy()
            if 1 <= j <= 5:
                h = r.integers(cfg.hidden)
                row[h] = np.uint16(int(row[h]) + (1 if r.random() < 0.5 else -1))
            wr[8 * grp + j] = row
        wr[8 * grp + 6] = wr[8 * grp + 7] = wr[8 * grp]
    ids = check(LayerData(cfg, 2, 0, 64, wr=wr)).cpu().numpy()
    for row in ids:  # a copy (6 or 7 in its group) comes only after the group's row 0
        for j, e in enumerate(row):
            if e % 8 >= 6:
                assert e - e % 8 in row[:j]


def test_bounded_router_overflowing_and_tiny_rows():
    """Token rows scaled by 2^125 (squared norm overflows fp32: every expert
    is recomputed) and by 2^-120 (products below fp32's normal range: the
    absolute term of the bound keeps every expert a candidate)."""
    cfg = C2
    T = 40
    x = synth.activations(cfg, 0, 4, T).view(np.uint16).reshape(T, cfg.hidden)
    xf = (x.astype(np.uint32) << 16).view(np.float32).copy()
    xf[0:3] *= np.float32(2.0 ** 125)
    xf[5:9] *= np.float32(2.0 ** -120)
    assert np.isfinite(xf).all()
    check(LayerData(cfg, 4, 0, T, x=synth.f32_to_bf16_bits(xf)))


def test_bounded_router_with_selection_bias():
    cfg = C3
    T = 96
    bias = np.random.default_rng(21).normal(0.0, 0.05, (T, cfg.n_experts))
    check(LayerData(cfg, 1, 3, T), bias=bias)


def test_bounded_router_full_prefill_chunk():
    """The 8,192-token prefill chunk the benchmark routes (no logits output):
    every token's ids against the oracle and the fp64 path."""
    print("bounded route prefill chunk T=8192", flush=True)
    check(LayerData(C4, 0, 0, 8192))
