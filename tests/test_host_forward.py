"""The host leg of decode co-execution (ft_moe_forward_host) on the CPU
against the fp64 oracle: fp32, bf16, MXFP4 and NVFP4-like records, masks,
partition sums, repeated ids.  No GPU: the call reads host memory only.

Bar: max relative error 1e-5 (fp32 arithmetic on exactly decoded weights)."""
import numpy as np
import pytest

from oracle.moe import experts_forward, route, to_f64
from oracle.record import decode_record
from sparse_moe_expert_softmax_amd import ftmoe, synth
from sparse_moe_expert_softmax_amd.configs import BF16, C1, MXFP4, NVFP4, MoEConfig

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

SMALL_BF16 = MoEConfig("host_bf16", 120, hidden=512, inter=256, n_experts=16, top_k=4, act_dtype=BF16,
                       router_dtype=BF16, w_dtype=BF16, n_layers=1)
SMALL_MX = MoEConfig("host_mxfp4", 121, hidden=256, inter=384, n_experts=12, top_k=3, act_dtype=BF16,
                     router_dtype=BF16, w_dtype=MXFP4, n_layers=1)
SMALL_NV = MoEConfig("host_nvfp4", 122, hidden=384, inter=256, n_experts=10, top_k=4, act_dtype=BF16,
                     router_dtype=BF16, w_dtype=NVFP4, n_layers=1)


def _max_rel(got, ref):
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def _layer(cfg, T, seed):
    if not __import__("os").path.exists(ftmoe.LIB_PATH):
        pytest.skip("library not built")
    x = synth.activations(cfg, seed, 0, T)
    wr = synth.router_weights(cfg, 0)
    ids, gates, _ = route(to_f64(x, cfg.act_dtype), to_f64(wr, cfg.router_dtype), cfg.top_k)
    recs = synth.layer_records(cfg, 0)
    dec = {e: decode_record(recs[e], cfg.hidden, cfg.inter, cfg.w_dtype) for e in range(cfg.n_experts)}
    return x, ids.astype(np.int32), gates.astype(np.float32), recs, dec


def _host(cfg, x, ids, gates, recs, mask=None, threads=3, records=None):
    desc = ftmoe.make_desc(cfg)
    out = np.full((x.shape[0], cfg.hidden), np.nan, dtype=np.float32)
    ptrs = records if records is not None else [recs[e].ctypes.data for e in range(cfg.n_experts)]
    ftmoe.ft_moe_forward_host(desc, np.ascontiguousarray(x), np.ascontiguousarray(ids),
                              np.ascontiguousarray(gates), ptrs, out,
                              expert_mask=None if mask is None else np.asarray(mask, dtype=np.uint32),
                              n_threads=threads)
    return out


@pytest.mark.parametrize("cfg,T", [(C1, 16), (SMALL_BF16, 3), (SMALL_MX, 5), (SMALL_NV, 4)])
def test_host_forward_matches_oracle_with_masks(cfg, T):
    x, ids, gates, recs, dec = _layer(cfg, T, 3)
    x64 = to_f64(x, cfg.act_dtype)
    full = _host(cfg, x, ids, gates, recs)
    ref = experts_forward(x64, ids, gates.astype(np.float64), dec.__getitem__)
    assert _max_rel(full, ref) <= 1e-5
    words = (cfg.n_experts + 31) // 32
    m = (np.random.default_rng(9).integers(0, 2 ** 32, size=words, dtype=np.uint64)).astype(np.uint32)
    comp = (~m).astype(np.uint32)
    a = _host(cfg, x, ids, gates, recs, mask=m)
    b = _host(cfg, x, ids, gates, recs, mask=comp)
    ra = experts_forward(x64, ids, gates.astype(np.float64), dec.__getitem__, mask=m)
    assert _max_rel(a, ra) <= 1e-5
    assert _max_rel(a + b, full) <= 1e-6
    # one thread gives the same bits: every sum runs in a fixed order
    assert np.array_equal(_host(cfg, x, ids, gates, recs, threads=1), full)
    # the portable loops (negative thread count) agree with the SIMD ones
    assert _max_rel(_host(cfg, x, ids, gates, recs, threads=-2), full) <= 1e-6


def test_host_forward_reads_only_the_kept_experts_and_repeats_add():
    cfg, T = SMALL_MX, 4
    x, ids, gates, recs, dec = _layer(cfg, T, 5)
    ids = ids.copy()
    ids[1, 2] = ids[1, 0]
    keep = sorted(set(ids[:2].ravel().tolist()))
    m = np.zeros(1, dtype=np.uint32)
    for e in keep:
        m[0] |= np.uint32(1 << e)
    ptrs = [recs[e].ctypes.data if e in keep else 0 for e in range(cfg.n_experts)]
    got = _host(cfg, x, ids, gates, recs, mask=m, records=ptrs)
    ref = experts_forward(to_f64(x, cfg.act_dtype), ids, gates.astype(np.float64), dec.__getitem__, mask=m)
    assert _max_rel(got, ref) <= 1e-5
    with pytest.raises(ftmoe.FtError) as ei:   # a needed record is missing
        _host(cfg, x, ids, gates, recs, records=ptrs)
    assert ei.value.status == ftmoe.FT_EINVAL
