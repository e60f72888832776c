"""Pins of the fp64 oracle against things other than itself: format
definitions and torch's own fp8 / bf16 types, exact arithmetic (mpmath,
fractions), brute-force enumeration, closed forms, a dense all-experts
evaluation, torch's silu, and a second, independently written LRU."""
import itertools
import math
from collections import OrderedDict
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

from oracle import formats, mx
from oracle import moe as moe_mod
from oracle.lru import LruSim
from oracle.moe import exact_logits_row, mask_has, moe_layer, route, select_topk, silu, swiglu_expert
from oracle.record import decode_record
from sparse_moe_expert_softmax_amd import synth
from sparse_moe_expert_softmax_amd.configs import BF16, F32, MXFP4, NVFP4

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ------------------------------------------------------------------ formats --
def test_e2m1_all_codes_match_spec_table():
    spec = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]       # OCP MX v1.0 FP4 E2M1 values
    got = formats.e2m1_to_f64(np.arange(16))
    np.testing.assert_array_equal(got[:8], spec)
    np.testing.assert_array_equal(got[8:], [-v for v in spec])
    assert [formats.e2m1_scalar(c) for c in range(16)] == list(got)


def test_e8m0_all_codes():
    got = formats.e8m0_to_f64(np.arange(256))
    for v in range(255):
        assert got[v] == math.ldexp(1.0, v - 127)
    assert np.isnan(got[255])
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    np.testing.assert_array_equal(got[:255], ref[:255])


def test_e4m3_all_codes_match_torch():
    got = formats.e4m3_to_f64(np.arange(256))
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_bf16_decode_matches_torch():
    bits = np.random.default_rng(0).integers(0, 2 ** 16, 5000).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]   # finite only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(formats.bf16_bits_to_f64(bits), ref)


def test_nibble_order_hand_packed():
    # byte 0x21: element 0 = low nibble 1 (0.5), element 1 = high nibble 2 (1.0)
    # byte 0xF7: element 2 = 7 (6.0), element 3 = 0xF (-6.0)
    codes = formats.unpack_nibbles(np.array([0x21, 0xF7], dtype=np.uint8), 4)
    np.testing.assert_array_equal(formats.e2m1_to_f64(codes), [0.5, 1.0, 6.0, -6.0])


def test_mxfp4_record_hand_example():
    # H=32, I=32: one 32-block per row; fill gate row 0 by hand, everything else zero
    H = I = 32
    stride = synth.record_stride(H, I, MXFP4)
    rec = np.zeros(stride, dtype=np.uint8)
    rec[0] = 0x3A          # elements 0, 1 = codes 0xA (-1.0) and 0x3 (1.5)
    n = 3 * H * I
    scale_base = n // 2
    rec[scale_base + 0] = 127 + 3     # gate row 0 scale 2^3
    rec[scale_base + I * H // 32] = 127   # up row 0 scale 1 (codes zero)
    G, U, D = decode_record(rec, H, I, MXFP4)
    assert G[0, 0] == -8.0 and G[0, 1] == 12.0 and np.count_nonzero(G) == 2
    assert np.count_nonzero(U) == 0 and np.count_nonzero(D) == 0


def test_nvfp4_record_hand_example():
    H = I = 16
    stride = synth.record_stride(H, I, NVFP4)
    rec = np.zeros(stride, dtype=np.uint8)
    n = 3 * H * I
    rec[n // 2 + (H * I // 16) * 2 + (H // 16) * 5] = 0x38      # down row 5 block scale: E4M3 0x38 = 1.0
    rec[(2 * I * H) // 2 + (5 * I) // 2] = 0x07                   # down row 5 element 0 = 6.0
    ts = np.array([1.0, 1.0, 0.25], dtype="<f4").view(np.uint8)
    off = n // 2 + n // 16
    rec[off: off + 12] = ts
    G, U, D = decode_record(rec, H, I, NVFP4)
    assert D[5, 0] == 1.5 and np.count_nonzero(D) == 1
    assert np.count_nonzero(G) == 0 and np.count_nonzero(U) == 0


@pytest.mark.parametrize("wd", [F32, BF16, MXFP4, NVFP4])
def test_record_roundtrip_close_to_draws(wd):
    from sparse_moe_expert_softmax_amd.configs import MoEConfig
    cfg = MoEConfig("t", 99, hidden=64, inter=96, n_experts=2, top_k=1, act_dtype=F32,
                    router_dtype=F32, w_dtype=wd, n_layers=1)
    mats = synth.expert_fp32(cfg, 0, 1)
    dec = decode_record(synth.expert_record(cfg, 0, 1), 64, 96, wd)
    tol = {F32: 0, BF16: 2 ** -8, MXFP4: 0.35, NVFP4: 0.35}[wd]
    for m, d in zip(mats, dec):
        assert d.shape == m.shape
        if tol == 0:
            np.testing.assert_array_equal(d, m.astype(np.float64))
        else:
            rel = np.abs(d - m).max() / np.abs(m).max()
            assert rel <= tol


# -------------------------------------------------------------- mx (MXFP8) --
def test_mxfp8_scale_and_grid():
    g = np.random.default_rng(3)
    v = g.standard_normal(32 * 40) * np.exp2(g.integers(-20, 20, 32 * 40))
    q = mx.mxfp8_quantize(v)
    grid = formats.e4m3_to_f64(np.arange(0x7F))
    for b in range(0, v.size, 32):
        blk, qb = v[b:b + 32], q[b:b + 32]
        amax = np.abs(blk).max()
        X = math.floor(math.log2(amax)) - 8
        assert mx.mx_scale_exponent(blk) == X
        scaled = np.abs(qb) / 2.0 ** X
        assert np.all(np.isin(scaled, grid))          # every value on the E4M3 grid
        # nearest: no grid point strictly closer to |v|/2^X than the chosen one
        tgt = np.abs(blk) / 2.0 ** X
        err = np.abs(scaled - tgt)
        best = np.min(np.abs(grid[None, :] - np.minimum(tgt, 448.0)[:, None]), axis=1)
        assert np.all(err <= np.maximum(best, tgt - 448.0) + 1e-300)


def test_mxfp8_elements_match_torch_fp8_rounding():
    g = np.random.default_rng(5)
    v = g.standard_normal(32 * 64)
    q = mx.mxfp8_quantize(v)
    for b in range(0, v.size, 32):
        X = mx.mx_scale_exponent(v[b:b + 32])
        scaled = v[b:b + 32] / 2.0 ** X
        ok = np.abs(scaled) <= 448.0
        ref = torch.from_numpy(scaled[ok]).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        np.testing.assert_array_equal(q[b:b + 32][ok] / 2.0 ** X, ref)
        assert np.all(np.abs(q[b:b + 32][~ok]) / 2.0 ** X == 448.0)


def test_mxfp8_zero_block_and_ties():
    assert np.all(mx.mxfp8_quantize(np.zeros(32)) == 0)
    # block with amax 256 -> X = 0; 17 lies between 16 and 18 (step 2): tie -> even code 16
    v = np.zeros(32)
    v[0], v[1], v[2] = 256.0, 17.0, 19.0
    q = mx.mxfp8_quantize(v)
    assert q[0] == 256.0 and q[1] == 16.0 and q[2] == 20.0


def test_mxfp8_two_term_is_the_value_plus_its_quantised_residual():
    """Two terms: q1 is the one-term result; the second term is the one-term
    quantisation of v - q1 (so it sits on its own block's E4M3 grid).  Each
    term loses at most 1/8 of its block's largest magnitude (saturation at
    448 of a block scaled up to just under 512, or half a step of 3
    mantissa bits), so the sum is within 2^-6 of the block's largest
    magnitude; it is exact when v is already on the first term's grid."""
    g = np.random.default_rng(33)
    v = formats.bf16_bits_to_f64(synth.f32_to_bf16_bits(g.standard_normal(32 * 50).astype(np.float32)))
    two = mx.mxfp8_two_term(v)
    q1 = mx.mxfp8_quantize(v)
    r = v - q1
    np.testing.assert_array_equal(two - q1, mx.mxfp8_quantize(r))
    assert np.all(r.astype(np.float32).astype(np.float64) == r)   # the residual of a bf16 value is exact in fp32
    for b in range(0, v.size, 32):
        amax = np.abs(v[b:b + 32]).max()
        assert np.abs(v[b:b + 32] - two[b:b + 32]).max() <= 2.0 ** -6 * amax
    err1 = np.abs(v - q1).max() / np.abs(v).max()
    err2 = np.abs(v - two).max() / np.abs(v).max()
    assert err2 < err1 / 8
    exact = mx.mxfp8_quantize(g.standard_normal(64))
    np.testing.assert_array_equal(mx.mxfp8_two_term(exact), exact)
    h = g.standard_normal(64) * 3
    np.testing.assert_array_equal(mx.mxfp8_two_term_f32(h), mx.mxfp8_two_term(h.astype(np.float32).astype(np.float64)))


def test_bf16_round_matches_torch_including_ties_and_subnormals():
    """The oracle's bf16 rounding of y (8 significant bits, ties to even) against
    torch's fp32 -> bfloat16 conversion: random values over many binades, exact
    midpoints between neighbouring bf16 values, fp32 subnormals, overflow."""
    g = np.random.default_rng(11)
    v = g.standard_normal(20000) * np.exp2(g.integers(-130, 126, 20000))
    # exact midpoints: bf16 value b + half an ulp, for both parities of b
    base = formats.bf16_bits_to_f64(g.integers(0x0080, 0x7F7F, 4000, dtype=np.int64).astype(np.uint16))
    ulp = np.ldexp(1.0, np.frexp(base)[1] - 8)
    mids = base + 0.5 * ulp
    special = np.array([0.0, -0.0, 1e-40, -3e-45, 3.4e38, -3.4e38, np.inf, -np.inf, 1.0 + 2.0 ** -8,
                        1.0 + 3 * 2.0 ** -8])
    for arr in (v, mids, -mids, special):
        f32 = arr.astype(np.float32)
        ref = torch.from_numpy(f32).to(torch.bfloat16).to(torch.float64).numpy()
        got = mx.bf16_round_f32(arr)
        np.testing.assert_array_equal(got, ref)
    # a hand case: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> even (1.0)
    assert mx.bf16_round_f32(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert mx.bf16_round_f32(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


# ------------------------------------------------------------------ routing --
def _bf16_vals(shape, scale, seed):
    g = np.random.default_rng(seed)
    return formats.bf16_bits_to_f64(synth.f32_to_bf16_bits((g.standard_normal(shape) * scale).astype(np.float32)))


def test_exact_logits_match_mpmath():
    x = _bf16_vals((3, 512), 1.0, 1)
    w = _bf16_vals((5, 512), 0.02, 2)
    mpmath.mp.prec = 300
    for t in range(3):
        got = exact_logits_row(x[t], w)
        for e in range(5):
            ref = float(mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(b) for a, b in zip(x[t], w[e])))
            assert got[e] == ref


def test_exact_logits_survive_cancellation():
    x = np.array([[2.0 ** 60, 1.0, -(2.0 ** 60)]])
    w = np.array([[1.0, 1.0, 1.0], [0.0, 0.5, 0.0]])
    ids, gates, logits = route(x, w, 1)
    assert logits[0, 0] == 1.0 and ids[0, 0] == 0     # a naive left-to-right sum gives 0 < 0.5


def test_topk_matches_subset_enumeration():
    g = np.random.default_rng(7)
    for trial in range(200):
        E, k = 8, int(g.integers(1, 4))
        s = np.round(g.standard_normal(E), 1)            # coarse values -> frequent ties
        sel = list(select_topk(s, k))
        best = None
        for sub in itertools.combinations(range(E), k):
            rest = [e for e in range(E) if e not in sub]
            # a member must beat every non-member, equal scores going to the lower id
            if all((s[a] > s[b]) or (s[a] == s[b] and a < b) for a in sub for b in rest):
                assert best is None
                best = sub
        assert best is not None and sorted(sel) == list(best)
        # output order: score descending, id ascending
        for a, b in zip(sel, sel[1:]):
            assert s[a] > s[b] or (s[a] == s[b] and a < b)


def test_zero_router_ties_to_lowest_ids():
    x = _bf16_vals((4, 64), 1.0, 3)
    ids, gates, _ = route(x, np.zeros((16, 64)), 5)
    np.testing.assert_array_equal(ids, np.tile(np.arange(5), (4, 1)))
    np.testing.assert_allclose(gates, 0.2, rtol=0, atol=1e-15)


def test_duplicated_router_rows_tie_to_lower_id():
    x = _bf16_vals((6, 128), 1.0, 4)
    w = _bf16_vals((10, 128), 0.02, 5)
    w[7] = w[2]
    w[9] = w[2]
    ids, _, logits = route(x, w, 10)
    for t in range(6):
        r = list(ids[t])
        assert r.index(2) < r.index(7) < r.index(9)
        assert r.index(7) == r.index(2) + 1 and r.index(9) == r.index(2) + 2


def test_gate_closed_forms():
    x = _bf16_vals((8, 96), 1.0, 6)
    w = _bf16_vals((12, 96), 0.05, 7)
    ids, gates, logits = route(x, w, 4)
    np.testing.assert_allclose(gates.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    for t in range(8):
        l = logits[t, ids[t]]
        assert np.all(np.diff(l) <= 0)
        np.testing.assert_allclose(gates[t, 0] / gates[t, 1:], np.exp(l[0] - l[1:]), rtol=1e-13)
        # renormalised softmax == full softmax restricted and rescaled
        p = np.exp(logits[t] - logits[t].max())
        p /= p.sum()
        np.testing.assert_allclose(gates[t], p[ids[t]] / p[ids[t]].sum(), rtol=1e-13)
    ids1, g1, _ = route(x, w, 1)
    assert np.all(g1 == 1.0)
    _, g_raw, lg = route(x, w, 4, renormalize=False)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(g_raw, np.take_along_axis(p, ids, 1), rtol=1e-13)


def test_selection_bias_moves_selection_not_gates():
    x = _bf16_vals((4, 64), 1.0, 8)
    w = _bf16_vals((16, 64), 0.02, 9)
    want = np.array([[3, 5, 11], [0, 1, 2], [15, 7, 9], [4, 8, 12]])
    bias = np.zeros((4, 16))
    bias[np.arange(4)[:, None], want] = 30.0
    ids, gates, logits = route(x, w, 3, bias=bias)
    for t in range(4):
        assert sorted(ids[t]) == sorted(want[t])
        l = logits[t, ids[t]]
        np.testing.assert_allclose(gates[t], np.exp(l - l.max()) / np.exp(l - l.max()).sum(), rtol=1e-14)


def test_certified_blas_routing_equals_fsum_routing():
    T, E, H = 64, 32, 256
    x = _bf16_vals((T, H), 1.0, 10)
    w = _bf16_vals((E, H), 0.02, 11)
    w[5] = w[17]          # exact ties force the exact fallback
    ids_a, g_a, _ = route(x, w, 6, exact_all=True)
    ids_b, g_b, _ = route(x, w, 6, exact_all=False)
    np.testing.assert_array_equal(ids_a, ids_b)
    np.testing.assert_allclose(g_a, g_b, rtol=0, atol=1e-12)


def _adversarial_layer():
    """k=2 over 8 experts, x = ones.  Expert 7's router row cancels to an
    exact logit of 2.25, true rank 2 (ahead of expert 1's 2.0), but its terms
    are +-2^42, so the classical bound on a floating-point sum of that row is
    large (about 4): an approximate product may legitimately report it far
    lower.  Every value is an fp32 number and every product is exact."""
    H = 64
    x = np.ones((1, H))
    w = np.zeros((8, H))
    w[0, 0], w[1, 0], w[2, 0], w[3, 0] = 3.0, 2.0, 1.0, float(np.float32(0.9))
    w[4, 0], w[5, 0], w[6, 0] = 0.5, 0.4, 0.3
    w[7, :62] = np.where(np.arange(62) % 2 == 0, 2.0 ** 42, -(2.0 ** 42))
    w[7, 62] = 2.25
    return x, w


def _perturbed_approx(delta):
    """An approximate product that errs by `delta` [E] on every token, each
    entry inside the error bound it reports."""
    original = moe_mod.approx_logits

    def approx(x, wr):
        logits, bound = original(x, wr)
        assert np.all(np.abs(delta) <= bound)
        return logits + delta, bound
    return approx


def test_certification_checks_every_unselected_expert(monkeypatch):
    """An unselected expert whose error interval reaches above the k-th
    selected one blocks certification, however far down the approximate
    ranking puts it.  Comparing only neighbours in the approximate top k+1
    would certify {0, 1} here, while the exact top-2 is {0, 7}."""
    x, w = _adversarial_layer()
    ids_x, g_x, l_x = route(x, w, 2, exact_all=True)
    assert list(ids_x[0]) == [0, 7] and l_x[0, 7] == 2.25
    delta = np.zeros(8)
    delta[7] = -1.6                     # approximate logit 0.65: rank 5
    _, bound = moe_mod.approx_logits(x, w)
    assert bound[0, 7] > 1.6 > 100 * bound[0, :7].max()
    monkeypatch.setattr(moe_mod, "approx_logits", _perturbed_approx(delta))
    ids, gates, _ = route(x, w, 2, exact_all=False)
    np.testing.assert_array_equal(ids, ids_x)
    np.testing.assert_array_equal(gates, g_x)


def test_certified_tokens_take_gates_from_exact_logits(monkeypatch):
    """When the approximate order is certified, the gates still come from the
    correctly rounded logits of the selected experts, not the approximate
    ones: the gates equal the exact path's bit for bit."""
    T, E, H = 16, 32, 256
    x = _bf16_vals((T, H), 1.0, 21)
    w = _bf16_vals((E, H), 0.02, 22)
    ids_x, g_x, l_x = route(x, w, 6, exact_all=True)
    _, bound = moe_mod.approx_logits(x, w)
    g = np.random.default_rng(23)
    delta = (g.uniform(-1, 1, size=(T, E)) * bound * 0.5)
    def approx(xx, wr):
        logits, bnd = x @ w.T, bound
        return logits + delta, bnd
    monkeypatch.setattr(moe_mod, "approx_logits", approx)
    ids, gates, logits = route(x, w, 6, exact_all=False)
    np.testing.assert_array_equal(ids, ids_x)
    np.testing.assert_array_equal(gates, g_x)
    sel = np.take_along_axis(logits, ids, 1)
    np.testing.assert_array_equal(sel, np.take_along_axis(l_x, ids_x, 1))


def test_certification_rule_is_sound_on_random_intervals():
    """Brute force over random score intervals: whenever the rule certifies,
    every choice of exact scores inside the intervals (the end points
    included) gives the certified selection, in the certified order."""
    g = np.random.default_rng(24)
    accepted = 0
    for trial in range(3000):
        E, k = 6, int(g.integers(1, 4))
        s = np.round(g.standard_normal(E), 1)
        slack = g.uniform(0, 0.3, size=E) * (g.random(E) < 0.7)
        order = moe_mod.certified_order(s, slack, k)
        if order is None:
            continue
        accepted += 1
        for _ in range(20):
            true = s + slack * g.choice([-1.0, 1.0, 0.0], size=E) * g.random(E)
            np.testing.assert_array_equal(select_topk(true, k), order)
        for corner in itertools.product([-1.0, 1.0], repeat=E):
            true = s + slack * np.array(corner)
            np.testing.assert_array_equal(select_topk(true, k), order)
    assert accepted > 300


# ------------------------------------------------------------- expert FFN --
def test_single_expert_is_textbook_swiglu():
    g = np.random.default_rng(12)
    T, H, I = 5, 48, 80
    x = g.standard_normal((T, H))
    Gm, Um, Dm = g.standard_normal((I, H)) * .2, g.standard_normal((I, H)) * .2, g.standard_normal((H, I)) * .2
    xt = torch.from_numpy(x)
    ref = (torch.nn.functional.silu(xt @ torch.from_numpy(Gm).T) * (xt @ torch.from_numpy(Um).T)) @ torch.from_numpy(Dm).T
    out, ids, gates = moe_layer(x, np.zeros((1, H)), lambda e: (Gm, Um, Dm), 1)
    assert np.all(ids == 0) and np.all(gates == 1.0)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-13, atol=1e-13)
    assert np.allclose(silu(np.array([0.0, 1.0, -1.0])), [0.0, 1 / (1 + math.exp(-1)), -1 / (1 + math.e)])


def test_zero_up_and_linearity_in_down():
    g = np.random.default_rng(13)
    H, I = 32, 40
    x = g.standard_normal(H)
    Gm, Um, Dm = g.standard_normal((I, H)), g.standard_normal((I, H)), g.standard_normal((H, I))
    assert np.all(swiglu_expert(x, Gm, np.zeros_like(Um), Dm) == 0)
    np.testing.assert_allclose(swiglu_expert(x, Gm, Um, 2.5 * Dm), 2.5 * swiglu_expert(x, Gm, Um, Dm), rtol=1e-14)


# --------------------------------------------------------- whole layer ----
def _dense_bruteforce(x, wr, experts, k, mask=None, bias=None):
    """Every expert on every token, then a membership test by rank counting with
    exact rational logits, full-softmax gates renormalised over the members."""
    T, H = x.shape
    E = wr.shape[0]
    G = np.stack([experts(e)[0] for e in range(E)])
    U = np.stack([experts(e)[1] for e in range(E)])
    D = np.stack([experts(e)[2] for e in range(E)])
    a = np.einsum("eih,th->tei", G, x)
    b = np.einsum("eih,th->tei", U, x)
    Y = np.einsum("ehi,tei->teh", D, a / (1 + np.exp(-a)) * b)
    out = np.zeros((T, H))
    for t in range(T):
        lq = [sum((Fraction(float(xv)) * Fraction(float(wv)) for xv, wv in zip(x[t], wr[e])), Fraction(0))
              for e in range(E)]
        sq = [lq[e] + Fraction(0 if bias is None else float(bias[t, e])) for e in range(E)]
        l = np.array([float(v) for v in lq])
        p = np.exp(l - l.max())
        member = [sum(1 for f in range(E) if sq[f] > sq[e] or (sq[f] == sq[e] and f < e)) < k for e in range(E)]
        denom = sum(p[e] for e in range(E) if member[e])
        for e in range(E):
            if member[e] and mask_has(mask, e):
                out[t] += p[e] / denom * Y[t, e]
    return out


def _tiny_layer(seed, T=6, H=32, I=24, E=6):
    g = np.random.default_rng(seed)
    x = _bf16_vals((T, H), 1.0, seed)
    wr = _bf16_vals((E, H), 0.3, seed + 1)
    mats = [(g.standard_normal((I, H)) * .2, g.standard_normal((I, H)) * .2, g.standard_normal((H, I)) * .2)
            for _ in range(E)]
    return x, wr, (lambda e: mats[e])


@pytest.mark.parametrize("seed", [20, 21, 22])
def test_sparse_layer_equals_dense_bruteforce(seed):
    x, wr, ex = _tiny_layer(seed)
    for k in (1, 2, 3, 6):
        out, ids, gates = moe_layer(x, wr, ex, k)
        np.testing.assert_allclose(out, _dense_bruteforce(x, wr, ex, k), rtol=1e-12, atol=1e-12)
    bias = np.zeros((6, 6))
    bias[:, 4] = 5.0
    out, ids, gates = moe_layer(x, wr, ex, 2, bias=bias)
    assert np.all(ids[:, 0] == 4)
    np.testing.assert_allclose(out, _dense_bruteforce(x, wr, ex, 2, bias=bias), rtol=1e-12, atol=1e-12)


def test_masked_layer_equals_dense_bruteforce_and_partitions_sum():
    x, wr, ex = _tiny_layer(30, E=8)
    g = np.random.default_rng(31)
    full, _, _ = moe_layer(x, wr, ex, 3)
    for _ in range(6):
        bits = g.integers(0, 2, 8)
        m = synth.bits_to_mask(bits)[0]
        mc = synth.bits_to_mask(1 - bits)[0]
        part, _, _ = moe_layer(x, wr, ex, 3, mask=m)
        comp, _, _ = moe_layer(x, wr, ex, 3, mask=mc)
        np.testing.assert_allclose(part, _dense_bruteforce(x, wr, ex, 3, mask=m), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(part + comp, full, rtol=1e-12, atol=1e-12)
    none, _, _ = moe_layer(x, wr, ex, 3, mask=np.zeros(1, dtype=np.uint32))
    assert np.all(none == 0)


def test_repeated_expert_in_a_token_adds_each_term():
    """A token listing expert e twice with gates a and b gets (a + b) y_e."""
    g = np.random.default_rng(31)
    H, I = 16, 24
    mats = {e: (g.standard_normal((I, H)), g.standard_normal((I, H)), g.standard_normal((H, I))) for e in range(4)}
    x = g.standard_normal((2, H))
    ids = np.array([[3, 1, 3], [2, 2, 2]])
    gates = np.array([[0.5, 0.3, 0.2], [0.1, 0.6, 0.3]])
    out = moe_mod.experts_forward(x, ids, gates, mats.__getitem__)
    y = {e: swiglu_expert(x[t], *mats[e]) for t, e in ((0, 3), (0, 1))}
    np.testing.assert_allclose(out[0], 0.7 * y[3] + 0.3 * y[1], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(out[1], 1.0 * swiglu_expert(x[1], *mats[2]), rtol=1e-13, atol=1e-13)


def test_expert_major_order_gives_the_same_bits():
    """experts_forward_by_expert (each expert visited once) equals
    experts_forward bit for bit, with repeated ids, a mask, quantisation
    hooks and a subset of rows."""
    g = np.random.default_rng(32)
    T, H, I, E, k = 9, 32, 40, 6, 3
    mats = {e: (g.standard_normal((I, H)), g.standard_normal((I, H)), g.standard_normal((H, I))) for e in range(E)}
    x = g.standard_normal((T, H))
    ids = g.integers(0, E, size=(T, k))
    gates = g.random((T, k))
    mask = np.array([0b101101], dtype=np.uint32)
    q = lambda v: np.round(v * 8) / 8
    rows = [0, 2, 3, 7]
    a = moe_mod.experts_forward(x, ids, gates, mats.__getitem__, mask=mask, x_quant=q, h_quant=q, tokens=rows)
    b = moe_mod.experts_forward_by_expert(x, ids, gates, mats.__getitem__, rows, mask=mask, x_quant=q, h_quant=q)
    np.testing.assert_array_equal(a, b)


def test_identical_experts_give_plain_ffn():
    x, wr, _ = _tiny_layer(40)
    g = np.random.default_rng(41)
    mats = (g.standard_normal((24, 32)) * .2, g.standard_normal((24, 32)) * .2, g.standard_normal((32, 24)) * .2)
    out, _, _ = moe_layer(x, wr, lambda e: mats, 3)
    ref = np.stack([swiglu_expert(x[t], *mats) for t in range(x.shape[0])])
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)


def test_tiny_worked_example_closed_form():
    # H=2, I=1, E=3, k=2; x = (1, 0); router rows give logits (1, 0, -1)
    x = np.array([[1.0, 0.0]])
    wr = np.array([[1.0, 5.0], [0.0, 7.0], [-1.0, 3.0]])
    mats = {0: (np.array([[2.0, 0.]]), np.array([[3.0, 0.]]), np.array([[1.0], [-1.0]])),
            1: (np.array([[-1.0, 0.]]), np.array([[1.0, 0.]]), np.array([[0.5], [2.0]])),
            2: (np.array([[9.0, 9.]]), np.array([[9.0, 9.]]), np.array([[9.0], [9.0]]))}
    out, ids, gates = moe_layer(x, wr, lambda e: mats[e], 2)
    assert list(ids[0]) == [0, 1]
    g0 = math.e / (math.e + 1.0)
    g1 = 1.0 / (math.e + 1.0)
    h0 = 2.0 / (1 + math.exp(-2.0)) * 3.0            # silu(2) * 3
    h1 = -1.0 / (1 + math.exp(1.0)) * 1.0            # silu(-1) * 1
    want = g0 * h0 * np.array([1.0, -1.0]) + g1 * h1 * np.array([0.5, 2.0])
    np.testing.assert_allclose(out[0], want, rtol=1e-15, atol=1e-15)


# ---------------------------------------------------------------------- LRU --
class OrderedLru:
    """Second formulation: an ordered list of slots, least recently used first;
    slots used by one call are moved to the back in ascending slot order."""

    def __init__(self, L, E, S):
        self.E, self.S = E, S
        self.where = {}
        self.holder = {}
        self.order = OrderedDict((s, None) for s in range(S))

    def lookup(self, layer, ids):
        U = sorted(set(int(e) for e in ids))
        hits = [e for e in U if (layer, e) in self.where]
        misses = [e for e in U if (layer, e) not in self.where]
        if len(misses) > self.S - len(hits):
            return None
        used = [self.where[(layer, e)] for e in hits]
        for s in used:
            del self.order[s]
        victims = list(itertools.islice(self.order.keys(), len(misses)))
        for e, s in zip(misses, victims):
            del self.order[s]
            if s in self.holder:
                del self.where[self.holder[s]]
            self.holder[s] = (layer, e)
            self.where[(layer, e)] = s
        for s in sorted(used + victims):
            self.order[s] = None
        slot_ids = [self.where[(layer, int(e))] for e in ids]
        flags = [1 if int(e) in misses else 0 for e in ids]
        return slot_ids, flags, list(zip(misses, victims))


def test_lru_two_formulations_agree_on_random_traces():
    g = np.random.default_rng(50)
    for trial in range(400):
        L, E = int(g.integers(1, 4)), int(g.integers(2, 9))
        S = int(g.integers(1, L * E + 2))
        a, b = LruSim(L, E, S), OrderedLru(L, E, S)
        for call in range(int(g.integers(1, 40))):
            layer = int(g.integers(0, L))
            ids = g.integers(0, E, int(g.integers(1, 5)))
            ra, rb = a.lookup(layer, ids), b.lookup(layer, ids)
            if ra is None or rb is None:
                assert ra is None and rb is None
                continue
            np.testing.assert_array_equal(ra[0], rb[0])
            np.testing.assert_array_equal(ra[1], rb[1])
            assert ra[2] == rb[2]


def test_lru_textbook_closed_forms():
    n = 5
    sim = LruSim(1, n + 1, n)
    misses = 0
    for r in range(40):
        res = sim.lookup(0, [r % (n + 1)])
        misses += int(res[1][0])
    assert misses == 40                      # cycling n+1 keys through n slots: every access misses
    sim = LruSim(2, 8, 6)
    keys = [(0, 1), (1, 1), (0, 7), (1, 3), (0, 0), (1, 6)]
    seen, misses = set(), 0
    g = np.random.default_rng(51)
    for _ in range(200):
        l, e = keys[int(g.integers(0, 6))]
        misses += int(sim.lookup(l, [e])[1][0])
        seen.add((l, e))
    assert misses == len(seen)               # at most n keys: only first touches miss
    sim = LruSim(1, 4, 2)
    for e, want_slot in [(0, 0), (1, 1), (0, 0), (2, 1), (3, 0)]:
        assert sim.lookup(0, [e])[0][0] == want_slot   # 2 evicts 1 (LRU), 3 evicts 0


def test_lru_exhaustion_changes_nothing():
    sim = LruSim(2, 8, 4)
    sim.lookup(0, [1, 2])
    snap = sim.snapshot()
    assert sim.lookup(1, [0, 1, 2, 3, 4]) is None
    after = sim.snapshot()
    for u, v in zip(snap[:3], after[:3]):
        np.testing.assert_array_equal(u, v)
    assert snap[3] == after[3]
    res = sim.lookup(0, [1, 2, 5, 6])         # 2 hits + 2 misses into the 2 untouched slots
    assert sorted(s for _, s in res[2]) == [2, 3]


def test_lru_multi_key_call_rules():
    sim = LruSim(1, 10, 4)
    r = sim.lookup(0, [7, 3, 7, 9])
    # misses in ascending id take free slots in ascending order
    assert r[2] == [(3, 0), (7, 1), (9, 2)]
    assert list(r[0]) == [1, 0, 1, 2] and list(r[1]) == [1, 1, 1, 1]
    r = sim.lookup(0, [3, 4, 5])          # 3 hits; 4 -> free slot 3; 5 -> oldest (slot 1, tie by slot)
    assert r[2] == [(4, 3), (5, 1)] and list(r[1]) == [0, 1, 1]


def test_lru_snapshot_restore_replays_identically():
    g = np.random.default_rng(52)
    calls = [(int(g.integers(0, 3)), g.integers(0, 12, 3)) for _ in range(300)]
    a = LruSim(3, 12, 10)
    out_a = [a.lookup(l, ids) for l, ids in calls]
    b = LruSim(3, 12, 10)
    for l, ids in calls[:150]:
        b.lookup(l, ids)
    snap = b.snapshot()
    c = LruSim(3, 12, 10)
    c.restore(snap)
    for (l, ids), ref in zip(calls[150:], out_a[150:]):
        res = c.lookup(l, ids)
        np.testing.assert_array_equal(res[0], ref[0])
        assert res[2] == ref[2]
