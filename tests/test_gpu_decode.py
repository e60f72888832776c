"""GPU parity of the decode path against the fp64 oracle, through the C ABI.

Bars: routing ids, slot tables and miss flags bit-exact; gates within 1e-6;
outputs within max relative error 1e-5 (fp32 layer) / 1e-2 (bf16, MXFP4,
NVFP4-like layers); partition sums within 1e-5 of the unmasked output."""
import numpy as np
import pytest
import torch

from gpu_util import LayerData, dev, max_rel_err
from oracle.moe import experts_forward, to_f64
from oracle.lru import LruSim
from sparse_moe_expert_softmax_amd import ftmoe, synth
from sparse_moe_expert_softmax_amd.configs import C1, C2, C3, C5, MoEConfig, F32, BF16

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

TOL = {F32: 1e-5, BF16: 1e-2}


def tol(cfg):
    return 1e-5 if cfg.w_dtype == F32 else 1e-2


def check_route(ld: LayerData, bias=None):
    ids, gates, logits = ld.gpu_route(bias)
    torch.cuda.synchronize()
    o_ids, o_gates, o_logits = ld.oracle_route(bias)
    np.testing.assert_array_equal(ids.cpu().numpy(), o_ids)
    np.testing.assert_allclose(gates.cpu().numpy(), o_gates, rtol=0, atol=1e-6)
    np.testing.assert_allclose(logits.cpu().numpy(), o_logits, rtol=1e-9, atol=1e-12)
    return ids, gates, o_ids


def run_layer(cfg, layer, step, T, mask=None, x=None, wr=None):
    ld = LayerData(cfg, layer, step, T, x=x, wr=wr)
    ids, gates, o_ids = check_route(ld)
    ld.build_pool(o_ids.ravel())
    out = ld.gpu_forward(ids, gates, mask=mask).cpu().numpy()
    ref, _, _ = ld.oracle_layer(mask=mask)
    assert not np.isnan(out).any()
    err = max_rel_err(out, ref)
    assert err <= tol(cfg), f"max rel err {err:.3g} > {tol(cfg)}"
    return ld, ids, gates, out, ref


# --------------------------------------------------------------- routing --
@pytest.mark.parametrize("cfg,T", [(C1, 16), (C2, 4), (C3, 4), (C5, 4), (C1, 1), (C2, 37), (C1, 40), (C5, 70)])
def test_route_matches_oracle(cfg, T):
    print(f"route {cfg.name} T={T}", flush=True)
    check_route(LayerData(cfg, 0, 0, T))


@pytest.mark.parametrize("T", [4, 40])
def test_route_ties_zero_router_and_duplicate_rows(T):
    """Ties go to the lowest ids, at decode size (T <= 16) and on the
    many-token path (T > 16) alike."""
    cfg = C2
    ld = LayerData(cfg, 0, 1, T, wr=np.zeros((cfg.n_experts, cfg.hidden), dtype=np.uint16))
    ids, gates, _ = ld.gpu_route()
    np.testing.assert_array_equal(ids.cpu().numpy(), np.tile(np.arange(cfg.top_k), (T, 1)))
    np.testing.assert_allclose(gates.cpu().numpy(), 1.0 / cfg.top_k, rtol=0, atol=1e-7)
    wr = synth.router_weights(cfg, 3).copy()
    for dup in (17, 64, 101):
        wr[dup] = wr[5]
    x = synth.activations(cfg, 0, 3, 2 * T)
    # make expert 5 win for every token so its duplicates are selected too
    wr[5] = wr[17] = wr[64] = wr[101] = (synth.f32_to_bf16_bits(np.full(cfg.hidden, 0.0, np.float32)))
    x = x.copy()
    check_route(LayerData(cfg, 3, 0, 2 * T, x=x, wr=wr))


def test_route_selection_bias_follows_trace():
    cfg = C3
    tr = synth.zipf_trace(cfg, n_steps=2)[1, 7]              # [4, k]
    bias = synth.trace_bias(tr, cfg.n_experts)
    ld = LayerData(cfg, 7, 1, 4)
    ids, gates, o_ids = check_route(ld, bias=bias)
    for t in range(4):
        assert sorted(ids[t].cpu().tolist()) == sorted(tr[t].tolist())


# --------------------------------------------------------------- forward --
def test_forward_tiny_fp32():
    run_layer(C1, 0, 0, 16)


@pytest.mark.parametrize("T", [1, 5, 17, 33])
def test_forward_tiny_fp32_ragged(T):
    run_layer(C1, 0, T, T)


@pytest.mark.parametrize("b", [1, 2, 4])
@pytest.mark.parametrize("layer", [0, 39])
def test_forward_decode_bf16(b, layer):
    print(f"decode bf16 b={b} layer={layer}", flush=True)
    run_layer(C2, layer, 11 + layer, b)


def test_forward_deterministic_and_masks_partition():
    cfg = C2
    ld, ids, gates, out, ref = run_layer(cfg, 2, 5, 4)
    again = ld.gpu_forward(ids, gates).cpu().numpy()
    assert np.array_equal(out, again)                      # bitwise identical rerun
    masks = synth.partition_masks(cfg, 2, 4)
    full_words = (cfg.n_experts + 31) // 32
    for m in masks:
        comp = (~m) & np.uint32(0xFFFFFFFF)
        a = ld.gpu_forward(ids, gates, mask=m).cpu().numpy()
        b = ld.gpu_forward(ids, gates, mask=comp).cpu().numpy()
        assert max_rel_err(a + b, out) <= 1e-5
        ra, _, _ = ld.oracle_layer(mask=m)
        assert max_rel_err(a, ra) <= 1e-2
        rb, _, _ = ld.oracle_layer(mask=comp)
        assert max_rel_err(b, rb) <= 1e-2
    zero = ld.gpu_forward(ids, gates, mask=np.zeros(full_words, dtype=np.uint32)).cpu().numpy()
    assert np.all(zero == 0)


def test_forward_zero_tokens_is_noop():
    cfg = C1
    ld = LayerData(cfg, 0, 0, 0, x=np.zeros((0, cfg.hidden), np.float32))
    out = torch.zeros(1, dtype=torch.float32, device="cuda")
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    x = torch.zeros((0, cfg.hidden), dtype=torch.float32, device="cuda")
    pool = torch.zeros(256, dtype=torch.uint8, device="cuda")
    ftmoe.ft_moe_forward(ld.desc, x, ids, out, pool, out, ws)


def test_forward_mxfp4_decode():
    cfg = C3
    for b in (1, 4):
        print(f"mxfp4 b={b}", flush=True)
        run_layer(cfg, 5, 3, b)


@pytest.mark.parametrize("cfg,T", [(C3, 8), (C5, 6), (C5, 1), (C3, 10)])
def test_forward_fp4_decode_both_gate_up_paths(cfg, T):
    """fp4 gate/up has two loops: activations staged in LDS with block scales
    loaded four chunks at a time (when the token group's rows fit in 56 KB),
    and the per-chunk register loop otherwise. H4096 at 8 tokens and H6144
    at 6 tokens take the second; one token takes the first.  The down
    projection packs h's hi and lo terms into one product up to 8 tokens and
    takes a product each above (10 tokens x top-6 = 60 pairs)."""
    print(f"fp4 decode {cfg.name} T={T}", flush=True)
    run_layer(cfg, 2, 4, T)


def test_forward_nvfp4_decode_with_partition_masks():
    """The 753B-like NVFP4 layer at batch 4: for seeded 50/50 masks, each part
    against the oracle's masked output (max relative error 1e-2 of that
    part's own largest value), and part + complement against the unmasked
    output (1e-5)."""
    cfg = C5
    ld, ids, gates, out, ref = run_layer(cfg, 1, 2, 4)
    masks = synth.partition_masks(cfg, 1, 3)
    for m in masks:
        comp = (~m) & np.uint32(0xFFFFFFFF)
        a = ld.gpu_forward(ids, gates, mask=m).cpu().numpy()
        b = ld.gpu_forward(ids, gates, mask=comp).cpu().numpy()
        assert max_rel_err(a + b, out) <= 1e-5
        for part, mm in ((a, m), (b, comp)):
            r, _, _ = ld.oracle_layer(mask=mm)
            err = max_rel_err(part, r)
            assert err <= 1e-2, f"masked part: max rel err {err:.3g}"


def test_forward_rejects_bad_arguments():
    cfg = C2
    ld = LayerData(cfg, 0, 0, 2)
    ids, gates, _ = ld.gpu_route()
    ld.build_pool([])
    x = dev(ld.x)
    out = torch.empty((2, cfg.hidden), dtype=torch.float32, device="cuda")
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(ftmoe.FtError) as ei:
        ftmoe.ft_moe_forward(ld.desc, x, ids, gates, ld.pool, out, small)
    assert ei.value.status == ftmoe.FT_EWORKSPACE
    bad = ftmoe.make_desc(cfg)
    bad.top_k = cfg.n_experts + 1
    with pytest.raises(ftmoe.FtError) as ei:
        ftmoe.ft_moe_forward(bad, x, ids, gates, ld.pool, out, small)
    assert ei.value.status == ftmoe.FT_EINVAL


@pytest.mark.parametrize("cfg,T", [(C2, 2), (C3, 4), (C5, 3), (C2, 9), (C1, 5)])
def test_forward_repeated_expert_in_a_token(cfg, T):
    """ids given by the caller may list an expert twice for one token; each
    listing adds its own gated term, on the decode path (C2 T=2, C3 T=4, C5
    T=3), the general path (C2 T=9: 72 pairs) and the fp32 path alike."""
    print(f"repeated ids {cfg.name} T={T}", flush=True)
    ld = LayerData(cfg, 1, 3, T)
    g = np.random.default_rng(77 + T)
    k = cfg.top_k
    ids_np = np.stack([g.choice(cfg.n_experts, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    ids_np[0, k - 1] = ids_np[0, 0]                  # token 0: first expert again at the last rank
    if T > 1:
        ids_np[1, 1:] = ids_np[1, 0]                 # token 1: one expert at every rank
    gates_np = g.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    ld.build_pool(ids_np.ravel())
    out = ld.gpu_forward(dev(ids_np), dev(gates_np)).cpu().numpy()
    cache = {}

    def expert(e):
        if e not in cache:
            cache[e] = ld.experts_f64(e)
        return cache[e]

    ref = experts_forward(to_f64(ld.x, cfg.act_dtype), ids_np, gates_np.astype(np.float64), expert)
    err = max_rel_err(out, ref)
    assert err <= tol(cfg), f"max rel err {err:.3g}"


def test_forward_expert_listed_more_than_sixteen_times():
    """An expert listed at 24 of the 32 pairs (NVFP4 6144/2048/256/top-8, four
    tokens): its gate/up workgroups take the pairs in two groups of at most
    16 columns, and on the eight-wave staged loop (49 KB of staged rows) the
    second group stages the activation rows again after the first group's
    partials overwrote them."""
    cfg, T = C5, 4
    print(f"expert listed 24 times {cfg.name} T={T}", flush=True)
    ld = LayerData(cfg, 2, 5, T)
    g = np.random.default_rng(91)
    k = cfg.top_k
    ids_np = np.stack([g.choice(cfg.n_experts, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    ids_np[:3, :] = ids_np[0, 0]  # tokens 0-2: one expert at every rank
    gates_np = g.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    ld.build_pool(ids_np.ravel())
    out = ld.gpu_forward(dev(ids_np), dev(gates_np)).cpu().numpy()
    cache = {}

    def expert(e):
        if e not in cache:
            cache[e] = ld.experts_f64(e)
        return cache[e]

    ref = experts_forward(to_f64(ld.x, cfg.act_dtype), ids_np, gates_np.astype(np.float64), expert)
    err = max_rel_err(out, ref)
    assert err <= tol(cfg), f"max rel err {err:.3g}"


# ------------------------------------------------------------ slot table --
def _gpu_table(L, E, S):
    tb = torch.zeros(ftmoe.ft_slot_table_bytes(L, E, S), dtype=torch.uint8, device="cuda")
    ftmoe.ft_slot_table_init(tb, L, E, S)
    return tb


def _table_arrays(tb, L, E, S):
    a = tb.cpu().numpy().view(np.int32)
    tick = int(a[0])
    ks = a[16:16 + L * E].reshape(L, E)
    sk = a[16 + L * E:16 + L * E + S]
    lu = a[16 + L * E + S:16 + L * E + 2 * S].view(np.uint32)
    return tick, ks, sk, lu


def _lookup(tb, layer, ids_np):
    n = ids_np.size
    ids = dev(ids_np.astype(np.int32))
    slot = torch.empty(n, dtype=torch.int32, device="cuda")
    flags = torch.empty(n, dtype=torch.uint8, device="cuda")
    ml = torch.empty(2 * n, dtype=torch.int32, device="cuda")
    nm = torch.empty(1, dtype=torch.int32, device="cuda")
    ftmoe.ft_slot_lookup(tb, layer, ids, slot, flags, ml, nm)
    nmv = int(nm.item())
    return slot.cpu().numpy(), flags.cpu().numpy(), ml.cpu().numpy(), nmv


def test_slot_table_replays_lru_oracle_bit_exact():
    g = np.random.default_rng(60)
    for (L, E, S) in [(3, 16, 10), (2, 64, 24), (5, 8, 40)]:
        tb = _gpu_table(L, E, S)
        sim = LruSim(L, E, S)
        for call in range(300):
            layer = int(g.integers(0, L))
            ids = g.integers(0, E, int(g.integers(1, 9))).astype(np.int32)
            ref = sim.lookup(layer, ids)
            slot, flags, ml, nm = _lookup(tb, layer, ids)
            if ref is None:
                assert nm == -1
                continue
            np.testing.assert_array_equal(slot, ref[0])
            np.testing.assert_array_equal(flags, ref[1])
            assert nm == len(ref[2])
            assert [tuple(ml[2 * i:2 * i + 2]) for i in range(nm)] == [tuple(p) for p in ref[2]]
        tick, ks, sk, lu = _table_arrays(tb, L, E, S)
        assert tick == sim.tick
        np.testing.assert_array_equal(ks, sim.key_slot)
        np.testing.assert_array_equal(sk, sim.slot_key)
        np.testing.assert_array_equal(lu, sim.last_use)


def test_slot_table_exhaustion_changes_nothing():
    tb = _gpu_table(2, 16, 4)
    _lookup(tb, 0, np.array([1, 2], np.int32))
    before = [np.copy(v) if isinstance(v, np.ndarray) else v for v in _table_arrays(tb, 2, 16, 4)]
    slot, flags, ml, nm = _lookup(tb, 1, np.array([0, 1, 2, 3, 4], np.int32))
    assert nm == -1 and np.all(slot == -1)
    after = _table_arrays(tb, 2, 16, 4)
    assert before[0] == after[0]
    for u, v in zip(before[1:], after[1:]):
        np.testing.assert_array_equal(u, v)


def test_slot_table_zipf_trace_matches_oracle():
    cfg = C3
    L, E, S = cfg.n_layers, cfg.n_experts, cfg.n_slots
    tr = synth.zipf_trace(cfg, n_steps=48)
    for b in (1, 4):
        tb = _gpu_table(L, E, S)
        sim = LruSim(L, E, S)
        misses = 0
        for step in range(tr.shape[0]):
            for layer in range(L):
                ids = tr[step, layer, :b].ravel()
                ref = sim.lookup(layer, ids)
                slot, flags, ml, nm = _lookup(tb, layer, ids)
                np.testing.assert_array_equal(slot, ref[0])
                np.testing.assert_array_equal(flags, ref[1])
                assert nm == len(ref[2])
                misses += nm
        tick, ks, sk, lu = _table_arrays(tb, L, E, S)
        np.testing.assert_array_equal(ks, sim.key_slot)
        np.testing.assert_array_equal(lu, sim.last_use)
        assert misses > 0


def test_slot_table_full_zipf_trace_matches_oracle():
    """The whole 2,048-step x 43-layer Zipf(1.1) trace of the 284B-like
    layer, cold start, at batch 1 and batch 4: every lookup's slots, miss
    flags and miss list bit-exact against the LRU state machine, and the
    final table equal.  The device lookups run back to back (no host round
    trip between them) into one output array per batch."""
    cfg = C3
    L, E, S = cfg.n_layers, cfg.n_experts, cfg.n_slots
    tr = synth.zipf_trace(cfg)
    n_steps = tr.shape[0]
    assert n_steps == 2048
    for b in (1, 4):
        print(f"full trace b={b}: {n_steps} steps x {L} layers", flush=True)
        n = b * cfg.top_k
        tb = _gpu_table(L, E, S)
        ids_d = dev(np.ascontiguousarray(tr[:, :, :b].reshape(n_steps, L, n)).astype(np.int32))
        slot_d = torch.empty((n_steps, L, n), dtype=torch.int32, device="cuda")
        flag_d = torch.empty((n_steps, L, n), dtype=torch.uint8, device="cuda")
        ml_d = torch.empty((n_steps, L, 2 * n), dtype=torch.int32, device="cuda")
        nm_d = torch.empty((n_steps, L), dtype=torch.int32, device="cuda")
        for step in range(n_steps):
            for layer in range(L):
                ftmoe.ft_slot_lookup(tb, layer, ids_d[step, layer], slot_d[step, layer], flag_d[step, layer],
                                     ml_d[step, layer], nm_d[step, layer:layer + 1])
        torch.cuda.synchronize()
        slot, flag, ml, nm = (t.cpu().numpy() for t in (slot_d, flag_d, ml_d, nm_d))
        sim = LruSim(L, E, S)
        misses = 0
        for step in range(n_steps):
            for layer in range(L):
                ref = sim.lookup(layer, tr[step, layer, :b].ravel())
                np.testing.assert_array_equal(slot[step, layer], ref[0])
                np.testing.assert_array_equal(flag[step, layer], ref[1])
                m = len(ref[2])
                assert nm[step, layer] == m
                np.testing.assert_array_equal(ml[step, layer, :2 * m], np.asarray(ref[2], dtype=np.int32).ravel())
                misses += m
        tick, ks, sk, lu = _table_arrays(tb, L, E, S)
        assert tick == sim.tick
        np.testing.assert_array_equal(ks, sim.key_slot)
        np.testing.assert_array_equal(sk, sim.slot_key)
        np.testing.assert_array_equal(lu, sim.last_use)
        rate = misses / float(n_steps * L * n)
        print(f"  miss rate {rate:.3f} of selected experts", flush=True)
        assert 0.2 < rate < 0.5


# ----------------------------------------------------------------- upload --
def test_upload_copies_records_and_rejects_pageable():
    cfg = C3
    stride = synth.record_stride(cfg.hidden, cfg.inter, cfg.w_dtype)
    rb = synth.record_bytes(cfg.hidden, cfg.inter, cfg.w_dtype)
    recs = [synth.expert_record(cfg, 2, e) for e in (3, 9)]
    host = [torch.from_numpy(r).pin_memory() for r in recs]
    pool = torch.zeros((8, stride), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    ev = torch.cuda.Event()
    ftmoe.ft_expert_upload(pool, stride, rb, [5, 1], [h.data_ptr() for h in host], stream=side, done_event=ev)
    torch.cuda.current_stream().wait_event(ev)
    got = pool.cpu().numpy()
    assert np.array_equal(got[5, :rb], recs[0][:rb]) and np.array_equal(got[1, :rb], recs[1][:rb])
    assert not got[0].any()
    pageable = torch.from_numpy(recs[0].copy())
    with pytest.raises(ftmoe.FtError) as ei:
        ftmoe.ft_expert_upload(pool, stride, rb, [2], [pageable.data_ptr()])
    assert ei.value.status == ftmoe.FT_EINVAL


def test_fetch_copies_the_lookups_misses_on_the_device():
    """ft_expert_fetch after ft_slot_lookup: the missed records land in their
    slots byte for byte (records of 130,560 bytes: a full and a partial 64 KB
    chunk), nothing else changes; an all-hit call and an exhausted pool
    (count -1) copy nothing."""
    from sparse_moe_expert_softmax_amd.configs import MXFP4
    cfg = MoEConfig("fetch_mxfp4_h256_i320", 97, hidden=256, inter=320, n_experts=16, top_k=2, act_dtype=BF16,
                    router_dtype=BF16, w_dtype=MXFP4, n_layers=1)
    E, S = cfg.n_experts, 4
    stride = synth.record_stride(cfg.hidden, cfg.inter, cfg.w_dtype)
    rb = synth.record_bytes(cfg.hidden, cfg.inter, cfg.w_dtype)
    recs = [synth.expert_record(cfg, 0, e) for e in range(E)]
    host = [torch.from_numpy(r).pin_memory() for r in recs]
    layer_src = torch.tensor([h.data_ptr() for h in host], dtype=torch.int64, device="cuda")
    table = torch.zeros(ftmoe.ft_slot_table_bytes(1, E, S), dtype=torch.uint8, device="cuda")
    ftmoe.ft_slot_table_init(table, 1, E, S)
    pool = torch.full((S, stride), 0xA5, dtype=torch.uint8, device="cuda")
    slots = torch.empty(8, dtype=torch.int32, device="cuda")
    flags = torch.empty(8, dtype=torch.uint8, device="cuda")
    mlist = torch.empty(17, dtype=torch.int32, device="cuda")  # [n_miss, (e, slot) ...]

    def call(ids):
        i = torch.tensor(ids, dtype=torch.int32, device="cuda")
        ftmoe.ft_slot_lookup(table, 0, i, slots[:len(ids)], flags[:len(ids)], mlist[1:], mlist[:1])
        ftmoe.ft_expert_fetch(pool, stride, rb, E, S, layer_src, mlist[1:], mlist[:1], max_miss=len(ids))
        torch.cuda.synchronize()
        return mlist.cpu().numpy()

    m = call([3, 9, 3, 12])
    assert m[0] == 3
    got = pool.cpu().numpy()
    filled = set()
    for q in range(m[0]):
        e, sl = int(m[1 + 2 * q]), int(m[2 + 2 * q])
        assert np.array_equal(got[sl, :rb], recs[e][:rb]), (e, sl)
        assert (got[sl, rb:] == 0xA5).all()  # the stride padding is not written
        filled.add(sl)
    for sl in set(range(S)) - filled:
        assert (got[sl] == 0xA5).all()
    before = pool.clone()
    m = call([9, 12, 3, 3])  # all hits
    assert m[0] == 0 and torch.equal(pool, before)
    m = call([0, 1, 2, 4, 5])  # five misses, four slots: exhausted
    assert m[0] == -1 and torch.equal(pool, before)
    with pytest.raises(ftmoe.FtError) as ei:
        ftmoe.ft_expert_fetch(pool, stride, rb + 8, E, S, layer_src, mlist[1:], mlist[:1], max_miss=4)
    assert ei.value.status == ftmoe.FT_EINVAL


# hidden 3072 and 2176: (H / 16) x 2 = 384 and 272 down items on 256
# workgroups, so some workgroups hold two items side by side and the rest one
UNEVEN_MX = MoEConfig("decode_mxfp4_h3072_e16", 84, hidden=3072, inter=256, n_experts=16, top_k=4, act_dtype=BF16,
                      router_dtype=BF16, w_dtype=2, n_layers=1)
UNEVEN_NV = MoEConfig("decode_nvfp4_h2176_e24", 85, hidden=2176, inter=384, n_experts=24, top_k=6, act_dtype=BF16,
                      router_dtype=BF16, w_dtype=3, n_layers=1)


@pytest.mark.parametrize("cfg,T", [(UNEVEN_MX, 2), (UNEVEN_NV, 3), (UNEVEN_NV, 1)])
def test_forward_decode_down_items_uneven_over_workgroups(cfg, T):
    """The down projection runs a workgroup's items side by side; where the
    item count is not a multiple of the grid, some workgroups hold fewer
    items than others.  Outputs against the oracle, partition parts summing
    to the full output."""
    print(f"uneven down items {cfg.name} T={T}", flush=True)
    ld, ids, gates, out, ref = run_layer(cfg, 0, 6 + T, T)
    m = np.array([0x00A5A5A5], dtype=np.uint32)
    comp = (~m) & np.uint32(0xFFFFFFFF)
    a = ld.gpu_forward(ids, gates, mask=m).cpu().numpy()
    b = ld.gpu_forward(ids, gates, mask=comp).cpu().numpy()
    assert max_rel_err(a + b, out) <= 1e-5


@pytest.mark.parametrize("cfg,T", [(C2, 9), (C3, 11)])
def test_forward_general_path_above_decode_pairs(cfg, T):
    """More than 64 (token, rank) pairs: the permute + grouped GEMV path."""
    print(f"general path {cfg.name} T={T}", flush=True)
    run_layer(cfg, 3, 7, T)


@pytest.mark.parametrize("cfg,T", [(C2, 2), (C3, 1), (C5, 4)])
def test_forward_decode_path_slot_indirection_and_poison(cfg, T):
    """Records placed at arbitrary pool slots through slot_ids; a negative slot
    (failed lookup) turns that expert's outputs into NaN instead of a fault.
    C3 at one token and C5 at four run the fp4 gate/up kernel on eight waves
    (two tiles side by side), C2 on four."""
    print(f"slot indirection and poison {cfg.name} T={T}", flush=True)
    ld = LayerData(cfg, 4, 9, T)
    ids, gates, o_ids = check_route(ld)
    uniq = sorted(set(o_ids.ravel().tolist()))
    slot_of = {e: 3 + 2 * i for i, e in enumerate(uniq)}
    pool = torch.full((3 + 2 * len(uniq), ld.stride), 0xFF, dtype=torch.uint8, device="cuda")
    for e, s in slot_of.items():
        pool[s].copy_(torch.from_numpy(ld.record(e)))
    slots = torch.from_numpy(np.vectorize(slot_of.get)(o_ids).astype(np.int32)).cuda()
    out = ld.gpu_forward(ids, gates, slot_ids=slots, pool=pool).cpu().numpy()
    ref, _, _ = ld.oracle_layer()
    assert max_rel_err(out, ref) <= 1e-2
    bad = slots.clone()
    bad[0, 0] = -1
    e0 = int(o_ids[0, 0])
    bad[torch.from_numpy(o_ids == e0).cuda()] = -1
    out2 = ld.gpu_forward(ids, gates, slot_ids=bad, pool=pool).cpu().numpy()
    assert np.isnan(out2[0]).any()
