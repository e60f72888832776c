"""GPU parity of the prefill path (MXFP4 weights on scaled MFMA, activations
carried as MXFP8) against the fp64 oracle, in both activation modes: two
MXFP8 terms (the default) and one.

Each output is compared with the oracle that mirrors the kernels' storage
precisions (OCP MX rule, one or two terms, for x before gate/up and for h
before down; expert outputs y rounded to bf16 before the combine) and, in
the two-term mode, also with the oracle on the exact bf16 activations and
fp64 h (no mirroring).

Bars: routing ids bit-exact for every token; gates within 1e-6; outputs within
max relative error 1e-2 of the mirrored oracle, and in the two-term mode also
of the unmirrored one."""
import numpy as np
import pytest
import torch

from gpu_util import LayerData, dev, max_rel_err
from oracle.moe import experts_forward_by_expert, to_f64
from oracle.mx import bf16_round_f32, mxfp8_quantize, mxfp8_quantize_f32, mxfp8_two_term, mxfp8_two_term_f32
from oracle.record import decode_record
from sparse_moe_expert_softmax_amd import ftmoe, synth
from sparse_moe_expert_softmax_amd.configs import BF16, C4, MXFP4, MoEConfig

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

SMALL = MoEConfig("prefill_small_mxfp4", 90, hidden=256, inter=256, n_experts=8, top_k=2, act_dtype=BF16,
                  router_dtype=BF16, w_dtype=MXFP4, n_layers=1)


def mirror(terms):
    """The oracle's quantisation hooks for the kernels' activation mode."""
    if terms == 1:
        return dict(x_quant=mxfp8_quantize, h_quant=mxfp8_quantize_f32, y_quant=bf16_round_f32)
    return dict(x_quant=mxfp8_two_term, h_quant=mxfp8_two_term_f32, y_quant=bf16_round_f32)


def run_prefill(cfg, T, layer, step, sample=None, mask=None, terms=2):
    ld = LayerData(cfg, layer, step, T)
    ld.desc.act_terms = terms
    ids, gates, logits = ld.gpu_route()
    torch.cuda.synchronize()
    o_ids, o_gates, _ = ld.oracle_route()
    np.testing.assert_array_equal(ids.cpu().numpy(), o_ids)
    np.testing.assert_allclose(gates.cpu().numpy(), o_gates, rtol=0, atol=1e-6)
    rows = range(T) if sample is None else sample
    need = sorted(set(int(e) for t in rows for e in o_ids[t]))
    ld.build_pool(need)
    out = ld.gpu_forward(ids, gates, mask=mask).cpu().numpy()
    ref, _, _ = ld.oracle_layer(mask=mask, tokens=list(rows), **mirror(terms))
    rows = list(rows)
    err = max_rel_err(out[rows], ref[rows])
    assert not np.isnan(out[rows]).any()
    assert err <= 1e-2, f"max rel err {err:.3g}"
    if terms == 2:
        exact, _, _ = ld.oracle_layer(mask=mask, tokens=rows)
        e2 = max_rel_err(out[rows], exact[rows])
        assert e2 <= 1e-2, f"max rel err {e2:.3g} against bf16 x and fp64 h"
    return ld, ids, gates, out, ref, err


@pytest.mark.parametrize("terms", [2, 1])
@pytest.mark.parametrize("T", [256, 300, 1031])
def test_prefill_small_layer_all_outputs(T, terms):
    print(f"prefill small T={T} terms={terms}", flush=True)
    _, _, _, _, _, err = run_prefill(SMALL, T, 0, T, terms=terms)
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


@pytest.mark.parametrize("terms", [2, 1])
def test_prefill_full_chunk_routing_and_sampled_outputs(terms):
    cfg, T = C4, 8192
    print(f"prefill 8192 tokens, full layer shape, terms={terms}", flush=True)
    sample = [0, 1234, 5000, 8191]
    _, _, _, _, _, err = run_prefill(cfg, T, 2, 0, sample=sample, terms=terms)
    print(f"  sampled max rel err {err:.3g}")


MID = MoEConfig("prefill_mid_mxfp4", 91, hidden=512, inter=384, n_experts=16, top_k=4, act_dtype=BF16,
                router_dtype=BF16, w_dtype=MXFP4, n_layers=1)


@pytest.mark.parametrize("terms", [2, 1])
def test_prefill_k_tails_and_several_weight_tiles(terms):
    """H 512 (four 128-K steps: one full group of three plus a tail), I 384
    (three steps, no tail), two gate/up and two down weight tiles, ragged
    expert row counts over 777 tokens."""
    print(f"prefill mid T=777 terms={terms}", flush=True)
    _, _, _, _, _, err = run_prefill(MID, 777, 0, 3, terms=terms)
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


def test_prefill_failed_lookup_poisons_only_its_tokens():
    """A negative slot for one expert (a failed lookup) makes exactly the
    tokens routed to it NaN, reads nothing for it, and leaves every other
    token bitwise unchanged (both activation modes)."""
    cfg, T = SMALL, 320
    for terms in (2, 1):
        ld, ids, gates, out, _, _ = run_prefill(cfg, T, 0, 9, terms=terms)
        ids_np = ids.cpu().numpy()
        slots = ids_np.astype(np.int32).copy()         # identity slots
        victim = int(ids_np[0, 0])
        slots[ids_np == victim] = -1
        got = ld.gpu_forward(ids, gates, slot_ids=dev(slots)).cpu().numpy()
        hit = (ids_np == victim).any(axis=1)
        assert np.isnan(got[hit]).all(axis=1).all()
        assert np.array_equal(got[~hit], out[~hit])


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
    run_prefill(SPARSE, 300, 0, 17, terms=1)
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
    run_prefill(FAT, 1100, 0, 19, terms=1)
    counts = np.bincount(ids.cpu().numpy().ravel(), minlength=2)
    assert counts.min() > 512, counts
    print(f"  rows per expert {counts.tolist()}, max rel err {err:.3g}")


# ------------------------------------------------- full 8,192-token chunks --
def _route_bounded(ld, x):
    """The many-token router as the forward's callers use it (no logits
    output: bf16 matrix-core scores with a rounding bound, fp64 refinement)."""
    cfg, T = ld.cfg, x.shape[0]
    ids = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, cfg.top_k), dtype=torch.float32, device="cuda")
    ws = torch.empty(ftmoe.ft_route_workspace_bytes(ld.desc, T), dtype=torch.uint8, device="cuda")
    ftmoe.ft_moe_route(ld.desc, dev(x), dev(ld.wr), ids, gates, workspace=ws)
    return ids, gates


def _cover_all_experts(o_ids, E, seed):
    """Tokens, in a seeded random order, each kept if it routes to an expert no
    earlier kept token does, until every expert is covered."""
    order = np.random.default_rng(seed).permutation(o_ids.shape[0])
    seen, rows = set(), []
    for t in order:
        new = set(int(e) for e in o_ids[t]) - seen
        if new:
            rows.append(int(t))
            seen |= new
        if len(seen) == E:
            break
    assert len(seen) == E
    return sorted(rows)


def test_prefill_full_chunks_outputs_cover_every_expert():
    """The 284B-like MXFP4 layer (4,096 / 2,048 / 256 experts / top-6) with
    every expert resident, as one 8,192-token chunk and as the 16,384-token
    prompt in two such chunks, activations as two MXFP8 terms.  Routing (the
    bounded router) bit-exact on every token of both chunks; outputs on
    tokens chosen so that together they use all 256 experts (chunk 1), and
    on 8 tokens of chunk 2, run on the same pool and workspace, against the
    oracle with the two-term storage mirrored and against the oracle on the
    exact bf16 x and fp64 h.  Chunk 1 also runs with one MXFP8 term, against
    its mirrored oracle; its error against the exact one is reported (one
    term keeps 3 mantissa bits: about 5-6% of the output range)."""
    cfg, T, layer = C4, 8192, 2
    ld = LayerData(cfg, layer, 0, T)
    print("prefill full chunks: generating 256 expert records on the device", flush=True)
    pool = synth.device_layer_pool(torch, cfg, layer, ld.stride)
    fws = torch.empty(ftmoe.ft_moe_workspace_bytes(ld.desc, T), dtype=torch.uint8, device="cuda")
    chunks = [ld.x, synth.activations(cfg, 1, layer, T)]
    w64 = to_f64(ld.wr, cfg.router_dtype)
    from oracle.moe import route
    results = []
    for c, x in enumerate(chunks):
        ids, gates = _route_bounded(ld, x)
        out = torch.empty((T, cfg.hidden), dtype=torch.float32, device="cuda")
        ftmoe.ft_moe_forward(ld.desc, dev(x), ids, gates, pool, out, fws)
        out1 = None
        if c == 0:  # one MXFP8 term
            d1 = ftmoe.make_desc(cfg, ld.stride, act_terms=1)
            out1 = torch.empty((T, cfg.hidden), dtype=torch.float32, device="cuda")
            ftmoe.ft_moe_forward(d1, dev(x), ids, gates, pool, out1, fws)
        torch.cuda.synchronize()
        x64 = to_f64(x, cfg.act_dtype)
        o_ids, o_gates, _ = route(x64, w64, cfg.top_k)
        np.testing.assert_array_equal(ids.cpu().numpy(), o_ids)
        np.testing.assert_allclose(gates.cpu().numpy(), o_gates, rtol=0, atol=1e-6)
        print(f"  chunk {c + 1}: routing bit-exact on all {T} tokens", flush=True)
        results.append((x64, o_ids, o_gates, out.cpu().numpy(), None if out1 is None else out1.cpu().numpy()))
    rows1 = _cover_all_experts(results[0][1], cfg.n_experts, 41)
    rows2 = sorted(np.random.default_rng(42).choice(T, 8, replace=False).tolist())
    print(f"  chunk 1: {len(rows1)} tokens cover all {cfg.n_experts} experts", flush=True)

    def expert(e):
        return decode_record(pool[e].cpu().numpy(), cfg.hidden, cfg.inter, cfg.w_dtype)

    for c, rows in ((0, rows1), (1, rows2)):
        x64, o_ids, o_gates, out, out1 = results[c]
        assert not np.isnan(out[rows]).any()
        ref = experts_forward_by_expert(x64, o_ids, o_gates, expert, rows, **mirror(2))
        err = max_rel_err(out[rows], ref[rows])
        print(f"  chunk {c + 1}: max rel err {err:.3g} on {len(rows)} tokens (two terms, mirrored)", flush=True)
        assert err <= 1e-2
        few = rows if c == 1 else rows[:24]
        exact = experts_forward_by_expert(x64, o_ids, o_gates, expert, few)
        e2 = max_rel_err(out[few], exact[few])
        print(f"  chunk {c + 1}: max rel err {e2:.3g} on {len(few)} tokens against bf16 x and fp64 h", flush=True)
        assert e2 <= 1e-2
        if out1 is not None:
            few1 = rows[:24]
            r1 = experts_forward_by_expert(x64, o_ids, o_gates, expert, few1, **mirror(1))
            e1 = max_rel_err(out1[few1], r1[few1])
            d1 = max_rel_err(out1[few1], exact[few1])
            print(f"  chunk 1, one term: max rel err {e1:.3g} mirrored, {d1:.3g} against bf16 x and fp64 h",
                  flush=True)
            assert e1 <= 1e-2 and d1 <= 0.1
