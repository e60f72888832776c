"""GPU: the fused route + forward entry point against the two calls it
replaces (ft_moe_route, then ft_moe_forward with every expert at its own
slot) on the same inputs, bit for bit, and against the oracle.

At decode sizes whose gate/up grid (min(T k, E) experts x I/8 row tiles,
halved when two tiles share a workgroup) stays within 1,024 workgroups, the
selection runs inside the gate/up kernel; otherwise the entry point runs the
two calls in sequence.  Both branches are covered: the *_SM shapes below keep
several tokens, a selection bias, a partition mask and full-softmax gates on
the in-kernel branch, which takes layers of at most 128 experts."""
import numpy as np
import pytest
import torch

from gpu_util import LayerData, dev, max_rel_err, to_f64
from sparse_moe_expert_softmax_amd import ftmoe
from sparse_moe_expert_softmax_amd.configs import BF16, C1, C2, C3, C5, MXFP4, NVFP4, MoEConfig

pytestmark = pytest.mark.gpu

SMALL = MoEConfig("prefill_small_mxfp4", 90, hidden=256, inter=256, n_experts=8, top_k=2, act_dtype=BF16,
                  router_dtype=BF16, w_dtype=MXFP4, n_layers=1)
NORENORM = MoEConfig("decode_bf16_full_softmax", 94, hidden=512, inter=128, n_experts=40, top_k=3,
                     act_dtype=BF16, router_dtype=BF16, w_dtype=BF16, n_layers=1, renormalize=False)
# in-kernel selection at several tokens: 384 workgroups at T=3 (staged-activation loop)
MX_SM = MoEConfig("decode_mxfp4_h2048_e64", 86, hidden=2048, inter=256, n_experts=64, top_k=4, act_dtype=BF16,
                  router_dtype=BF16, w_dtype=MXFP4, n_layers=1)
# 1,024 workgroups at T=4, the largest grid that still selects in-kernel
NV_SM = MoEConfig("decode_nvfp4_h2048_e64", 87, hidden=2048, inter=256, n_experts=64, top_k=8, act_dtype=BF16,
                  router_dtype=BF16, w_dtype=NVFP4, n_layers=1)


def fused_vs_separate(cfg, T, step, bias=None, mask=None, x=None, wr=None):
    ld = LayerData(cfg, 0, step, T, x=x, wr=wr)
    ids, gates, _ = ld.gpu_route(bias=bias)
    ld.build_pool(ids.cpu().numpy().ravel())
    out = ld.gpu_forward(ids, gates, mask=mask)
    torch.cuda.synchronize()

    k = cfg.top_k
    f_ids = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    f_gates = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    f_out = torch.full((T, cfg.hidden), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(ftmoe.ft_moe_route_forward_workspace_bytes(ld.desc, T), dtype=torch.uint8, device="cuda")
    b = None if bias is None else dev(bias.astype(np.float32))
    m = None if mask is None else dev(np.asarray(mask, dtype=np.uint32))
    for _ in range(2):  # a second call on the same workspace gives the same results
        ftmoe.ft_moe_route_forward(ld.desc, dev(ld.x), dev(ld.wr), f_ids, f_gates, ld.pool, f_out, ws,
                                   sel_bias=b, expert_mask=m)
        torch.cuda.synchronize()
        assert torch.equal(f_ids, ids)
        assert torch.equal(f_gates.view(torch.int32), gates.view(torch.int32))
        assert torch.equal(f_out.view(torch.int32), out.view(torch.int32))
    return ld, f_ids, f_gates, f_out


@pytest.mark.parametrize("T", [1, 2, 4])
def test_fused_bf16_decode_matches_separate_calls(T):
    print(f"fused C2 T={T}", flush=True)
    fused_vs_separate(C2, T, 100 + T)


@pytest.mark.parametrize("cfg,T", [(C2, 1), (C3, 1), (C3, 3), (MX_SM, 3)])
def test_fused_mxfp4_decode_with_selection_bias(cfg, T):
    """(C2 at one token: the workgroup-wide ranking with a bias; C3 has 256
    experts, above the in-kernel selection's limit: the two calls.)"""
    print(f"fused {cfg.name} T={T} with selection bias", flush=True)
    bias = np.random.default_rng(3 + T).normal(0.0, 0.5, (T, cfg.n_experts))
    fused_vs_separate(cfg, T, 110 + T, bias=bias)


@pytest.mark.parametrize("cfg", [C5, NV_SM])
def test_fused_nvfp4_decode_with_partition_mask(cfg):
    print(f"fused {cfg.name} T=4 with mask", flush=True)
    m = np.array([0xA5A5A5A5, 0x0F0F0F0F, 0xFFFF0000, 0x12345678, 0x0, 0xFFFFFFFF, 0x3C3C3C3C, 0x55555555],
                 dtype=np.uint32)[:(cfg.n_experts + 31) // 32]
    ld, _, _, f_out = fused_vs_separate(cfg, 4, 120, mask=m)
    if cfg is NV_SM:  # the oracle layer at C5's size would decode 32 experts of 6144 x 2048 in fp64
        ref, _, _ = ld.oracle_layer(mask=m)
        assert max_rel_err(f_out.cpu().numpy(), ref) <= 1e-2


def test_fused_one_token_ranked_with_partition_masks():
    """One token ranked by the whole workgroup, with a partition mask (the
    grouping then takes the general path): each part against the separate
    calls bit for bit, the two parts summing to the full output."""
    cfg = C2
    print("fused C2 T=1 with masks", flush=True)
    m = np.array([0xF0F0F0F0, 0x0F0F0F0F, 0xAAAA5555, 0x12345678], dtype=np.uint32)
    ld, _, _, part_a = fused_vs_separate(cfg, 1, 160, mask=m)
    _, _, _, part_b = fused_vs_separate(cfg, 1, 160, mask=~m)
    _, _, _, full = fused_vs_separate(cfg, 1, 160)
    ref, _, _ = ld.oracle_layer()
    assert max_rel_err((part_a + part_b).cpu().numpy(), ref) <= 1e-3
    assert max_rel_err(full.cpu().numpy(), ref) <= 1e-3


def test_fused_full_softmax_gates_and_oracle():
    """renormalize off (gates are full-softmax probabilities), 16 tokens:
    the largest decode batch the fused kernel selects for."""
    print("fused full-softmax T=16", flush=True)
    ld, f_ids, f_gates, f_out = fused_vs_separate(NORENORM, 16, 130)
    o_ids, o_gates, _ = ld.oracle_route()
    np.testing.assert_array_equal(f_ids.cpu().numpy(), o_ids)
    np.testing.assert_allclose(f_gates.cpu().numpy(), o_gates, rtol=0, atol=1e-6)
    ref, _, _ = ld.oracle_layer()
    assert max_rel_err(f_out.cpu().numpy(), ref) <= 1e-3


def test_fused_one_token_ties_take_the_exact_rounds():
    """At one token the gate/up workgroup ranks the experts by the high 32
    bits of their keys.  Where those tie inside the top k it must hand over to
    the exact rounds: a zero router (every logit equal), and two experts whose
    logits differ only below the high half (one bf16 ulp of one router weight,
    times the smallest activation).  Both against the separate calls, bit for
    bit, and against the oracle's selection."""
    cfg = C2
    print("fused C2 T=1, zero router", flush=True)
    zero = np.zeros((cfg.n_experts, cfg.hidden), dtype=np.uint16)
    _, f_ids, f_gates, _ = fused_vs_separate(cfg, 1, 150, wr=zero)
    np.testing.assert_array_equal(f_ids.cpu().numpy(), np.arange(cfg.top_k)[None, :])
    np.testing.assert_allclose(f_gates.cpu().numpy(), 1.0 / cfg.top_k, rtol=0, atol=1e-7)

    print("fused C2 T=1, logits tied in their high 32 bits", flush=True)
    base = LayerData(cfg, 0, 151, 1)
    o_ids, _, o_logits = base.oracle_route()
    ea, eb = int(o_ids[0, 0]), int(o_ids[0, 2])
    x64 = to_f64(base.x, cfg.act_dtype)[0]
    w = base.wr.copy()
    w[eb] = w[ea]
    nz = np.flatnonzero((x64 != 0) & (to_f64(w[ea], cfg.router_dtype) != 0))
    j = int(nz[np.argmin(np.abs(x64[nz]))])
    w[eb, j] = w[ea, j] + 1  # one bf16 ulp away (same sign and exponent: the low mantissa bit)
    ld = LayerData(cfg, 0, 151, 1, wr=w)
    o_ids2, _, o_logits2 = ld.oracle_route()
    la, lb = np.float64(o_logits2[0, ea]), np.float64(o_logits2[0, eb])
    assert la != lb and (la.view(np.uint64) >> 32) == (lb.view(np.uint64) >> 32), (la, lb)
    _, f_ids, _, _ = fused_vs_separate(cfg, 1, 151, wr=w)
    np.testing.assert_array_equal(f_ids.cpu().numpy(), o_ids2)


@pytest.mark.parametrize("cfg,T", [(C1, 16), (SMALL, 300), (C2, 17), (C2, 12), (C5, 9)])
def test_unfused_sizes_run_the_two_calls(cfg, T):
    """fp32, many tokens, and decode-sized token counts whose T * k exceeds
    the 64 pairs the fused kernels group (12 x top-8, 9 x top-8 NVFP4)."""
    print(f"route+forward {cfg.name} T={T}", flush=True)
    fused_vs_separate(cfg, T, 140 + T)
