"""GPU parity of the prefill path (MXFP4 weights on scaled MFMA, activations
quantised to MXFP8) against the fp64 oracle with the same storage precisions
mirrored (OCP MX rule for x before gate/up and for h before down; expert
outputs y rounded to bf16 before the combine).

Bars: routing ids bit-exact for every token; gates within 1e-6; outputs within
max relative error 1e-2."""
import numpy as np
import pytest
import torch

from gpu_util import LayerData, max_rel_err
from oracle.mx import bf16_round_f32, mxfp8_quantize, mxfp8_quantize_f32
from sparse_moe_expert_softmax_amd.configs import BF16, C4, MXFP4, MoEConfig

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

SMALL = MoEConfig("prefill_small_mxfp4", 90, hidden=256, inter=256, n_experts=8, top_k=2, act_dtype=BF16,
                  router_dtype=BF16, w_dtype=MXFP4, n_layers=1)


def run_prefill(cfg, T, layer, step, sample=None, mask=None):
    ld = LayerData(cfg, layer, step, T)
    ids, gates, logits = ld.gpu_route()
    torch.cuda.synchronize()
    o_ids, o_gates, _ = ld.oracle_route()
    np.testing.assert_array_equal(ids.cpu().numpy(), o_ids)
    np.testing.assert_allclose(gates.cpu().numpy(), o_gates, rtol=0, atol=1e-6)
    rows = range(T) if sample is None else sample
    need = sorted(set(int(e) for t in rows for e in o_ids[t]))
    ld.build_pool(need)
    out = ld.gpu_forward(ids, gates, mask=mask).cpu().numpy()
    ref, _, _ = ld.oracle_layer(mask=mask, tokens=list(rows), x_quant=mxfp8_quantize, h_quant=mxfp8_quantize_f32,
                                y_quant=bf16_round_f32)
    rows = list(rows)
    err = max_rel_err(out[rows], ref[rows])
    assert not np.isnan(out[rows]).any()
    assert err <= 1e-2, f"max rel err {err:.3g}"
    return ld, ids, gates, out, ref, err


@pytest.mark.parametrize("T", [256, 300, 1031])
def test_prefill_small_layer_all_outputs(T):
    print(f"prefill small T={T}", flush=True)
    _, _, _, _, _, err = run_prefill(SMALL, T, 0, T)
    print(f"  max rel err {err:.3g}")


def test_prefill_small_layer_partition_masks():
    ld, ids, gates, out, ref, _ = run_prefill(SMALL, 384, 0, 5)
    m = np.array([0b10110010], dtype=np.uint32)
    comp = (~m) & np.uint32(0xFF)
    a = ld.gpu_forward(ids, gates, mask=m).cpu().numpy()
    b = ld.gpu_forward(ids, gates, mask=comp).cpu().numpy()
    assert max_rel_err(a + b, out) <= 1e-5
    again = ld.gpu_forward(ids, gates).cpu().numpy()
    assert np.array_equal(again, out)  # deterministic


def test_prefill_full_chunk_routing_and_sampled_outputs():
    cfg, T = C4, 8192
    print("prefill 8192 tokens, full layer shape", flush=True)
    sample = [0, 1234, 5000, 8191]
    _, _, _, _, _, err = run_prefill(cfg, T, 2, 0, sample=sample)
    print(f"  sampled max rel err {err:.3g}")


MID = MoEConfig("prefill_mid_mxfp4", 91, hidden=512, inter=384, n_experts=16, top_k=4, act_dtype=BF16,
                router_dtype=BF16, w_dtype=MXFP4, n_layers=1)


def test_prefill_k_tails_and_several_weight_tiles():
    """H 512 (four 128-K steps: one full group of three plus a tail), I 384
    (three steps, no tail), two gate/up and two down weight tiles, ragged
    expert row counts over 777 tokens."""
    print("prefill mid T=777", flush=True)
    _, _, _, _, _, err = run_prefill(MID, 777, 0, 3)
    print(f"  max rel err {err:.3g}")


def test_prefill_slot_indirection_matches_identity_slots():
    """The forward reads expert e at pool + slot_ids[pair] * stride: records
    moved to other slots give bitwise the same output."""
    cfg, T = SMALL, 320
    ld, ids, gates, out, _, _ = run_prefill(cfg, T, 0, 9)
    E = cfg.n_experts
    perm = np.random.default_rng(5).permutation(E)          # expert e lives in slot perm[e]
    pool2 = torch.full((E, ld.stride), 0xFF, dtype=torch.uint8, device="cuda")
    for e in range(E):
        pool2[perm[e]].copy_(ld.pool[e])
    slots = torch.from_numpy(perm[ids.cpu().numpy()].astype(np.int32)).cuda()
    moved = ld.gpu_forward(ids, gates, slot_ids=slots, pool=pool2).cpu().numpy()
    assert np.array_equal(moved, out)


def test_prefill_masked_out_experts_are_never_read():
    """Poison (NaN) the records of the masked-out experts: the masked output
    stays finite and equals the masked output over the intact pool."""
    cfg, T = SMALL, 300
    ld, ids, gates, _, _, _ = run_prefill(cfg, T, 0, 11)
    m = np.array([0b01011001], dtype=np.uint32)
    ref = ld.gpu_forward(ids, gates, mask=m).cpu().numpy()
    for e in range(cfg.n_experts):
        if not (int(m[0]) >> e) & 1:
            ld.pool[e].fill_(0xFF)
    got = ld.gpu_forward(ids, gates, mask=m).cpu().numpy()
    assert not np.isnan(got).any()
    assert np.array_equal(got, ref)


def test_prefill_threshold_general_path_below_256_tokens():
    """255 tokens take the general (fp32 GEMV) path with unquantised
    activations; 256 take the matrix cores. Both against the oracle."""
    cfg = SMALL
    ld = LayerData(cfg, 0, 13, 255)
    ids, gates, _ = ld.gpu_route()
    o_ids, _, _ = ld.oracle_route()
    np.testing.assert_array_equal(ids.cpu().numpy(), o_ids)
    ld.build_pool(o_ids.ravel())
    out = ld.gpu_forward(ids, gates).cpu().numpy()
    ref, _, _ = ld.oracle_layer()
    assert max_rel_err(out, ref) <= 1e-2
    run_prefill(cfg, 256, 0, 13)


SPARSE = MoEConfig("prefill_sparse_mxfp4", 92, hidden=768, inter=640, n_experts=128, top_k=2, act_dtype=BF16,
                   router_dtype=BF16, w_dtype=MXFP4, n_layers=1)


def test_prefill_sparse_experts_and_k_tails():
    """128 experts for 600 pairs: one expert without rows, the others with
    1-13 (so most waves of a row chunk hold no valid row), H 768 (six 128-K
    steps: two full scale groups, no tail) and I 640 (five steps: a partial
    scale group and a tail of five), five gate/up and three down weight tiles."""
    print("prefill sparse T=300", flush=True)
    _, ids, _, _, _, err = run_prefill(SPARSE, 300, 0, 17)
    counts = np.bincount(ids.cpu().numpy().ravel(), minlength=SPARSE.n_experts)
    assert counts.min() == 0 and counts.max() < 16, (counts.min(), counts.max())
    print(f"  max rel err {err:.3g}")


FAT = MoEConfig("prefill_fat_mxfp4", 93, hidden=256, inter=128, n_experts=2, top_k=1, act_dtype=BF16,
                router_dtype=BF16, w_dtype=MXFP4, n_layers=1)


def test_prefill_experts_spanning_several_row_chunks():
    """Two experts, top-1, 1,100 tokens: each expert's rows span three
    256-row chunks (the last one partial); the down projection has a single
    128-K step (I 128)."""
    print("prefill fat T=1100", flush=True)
    ld, ids, _, _, _, err = run_prefill(FAT, 1100, 0, 19)
    counts = np.bincount(ids.cpu().numpy().ravel(), minlength=2)
    assert counts.min() > 512, counts
    print(f"  rows per expert {counts.tolist()}, max rel err {err:.3g}")
