"""Benchmark of the MoE-layer hot path on one MI355X.

Default workload: decode MoE layer with hidden 2048, 128 experts, top-8,
expert intermediate 768, bf16 weights N(0, 0.02), bf16 activations N(0, 1),
40 layers of independent random weights resident in HBM (48.3 GB), batch 1
(also --batch 2 / 4).  One step = the whole layer stack once: for each of the
40 layers, route (fp64 logits, top-k, gates) then forward (permute, grouped
gate/up + SwiGLU GEMV, down GEMV, combine), with fresh activations for every
(step, layer).  The metric is MoE-layer tokens/s = batch * layers / step time.

Printed: one JSON line with the metric, a roofline object for the expert
forward (algorithmic bytes = the distinct experts each call actually routed
to, times their record bytes, plus activations in and fp32 outputs out, over
the forward's measured duration, against the 8 TB/s HBM peak), the same
figures at batches 2 and 4 (other_batches), the metric's prefill half (one
8,192-token chunk through the MXFP4 layer with its experts resident: route
and forward durations, tokens/s, matrix-core TFLOP/s against the issued fp8
rate and the MXFP4 peak, measured HBM traffic), and the fp64 oracle timed on
this host's cores on a bounded sample of the same decode workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# Measured HBM bytes per ft_moe_forward call of the default decode workload
# (bf16, H2048, E128, top-8, batch 1): rocprofv3 FETCH_SIZE and WRITE_SIZE of
# the two decode kernels per call, scaled by what the same counters read for a
# plain 256 MiB device copy (FETCH_SIZE x 1.9997, WRITE_SIZE x 1.0).  Keyed by
# one SHA-256 prefix over the kernel source and every header it includes: any
# change to them reports null until the counters are taken again.
_CSRC = os.path.join(ROOT, "sparse_moe_expert_softmax_amd", "csrc")
_HEADERS = [os.path.join(_CSRC, "common.hpp"), os.path.join(_CSRC, "internal.hpp"),
            os.path.join(ROOT, "include", "ft_moe.h")]
DECODE_SRCS = [os.path.join(_CSRC, f) for f in ("decode_mfma.hip", "topk.hpp")] + _HEADERS
DECODE_TRAFFIC = {"fb941ebdb53fa6d6": 75968138}
# The same for the prefill workloads (8,192-token chunks: MXFP4 H4096 E256
# top-6 in either activation mode, bf16 H2048 E128 top-8, NVFP4 H6144 E256
# top-8): every kernel of one ft_moe_forward call, keyed by the workload, the
# activation terms of the matrix-core path (1 for bf16 and NVFP4 weights) and
# the prefix over the sources the workload's kernels come from.
PREFILL_SRCS = {
    "prefill_mxfp4_h4096_e256": [os.path.join(_CSRC, f) for f in ("mfma.hip", "lds_dma.hpp", "permute.hip",
                                                                   "gemv.hip")] + _HEADERS,
    "prefill_bf16_h2048_e128": [os.path.join(_CSRC, f) for f in ("prefill_bf16.hip", "mfma.hip", "lds_dma.hpp",
                                                                  "permute.hip", "gemv.hip")] + _HEADERS,
    "prefill_nvfp4_h6144_e256": [os.path.join(_CSRC, f) for f in ("prefill_bf16.hip", "mfma.hip", "lds_dma.hpp",
                                                                   "permute.hip", "gemv.hip")] + _HEADERS,
}
PREFILL_WORKLOADS = tuple(PREFILL_SRCS)
PREFILL_TRAFFIC = {
    ("prefill_mxfp4_h4096_e256", 2, "fede5405306ea7b4"): 5699135373,
    ("prefill_mxfp4_h4096_e256", 1, "fede5405306ea7b4"): 4989481371,
    ("prefill_bf16_h2048_e128", 1, "7d8e1e5fe1ebc036"): 2705608519,
    ("prefill_nvfp4_h6144_e256", 1, "7d8e1e5fe1ebc036"): 10380571040,
}


def sources_hash(paths):
    """SHA-256 prefix (16 hex digits) over the files' bytes, in order."""
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_decode_traffic(cfg_name, batch):
    if cfg_name != "decode_bf16_h2048_e128" or batch != 1:
        return None
    return DECODE_TRAFFIC.get(sources_hash(DECODE_SRCS))


def measured_prefill_traffic(cfg_name, chunk_tokens, terms=2):
    if cfg_name not in PREFILL_WORKLOADS or chunk_tokens != 8192:
        return None
    if cfg_name != "prefill_mxfp4_h4096_e256":
        terms = 1
    return PREFILL_TRAFFIC.get((cfg_name, terms, sources_hash(PREFILL_SRCS[cfg_name])))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--single-batch", action="store_true",
                    help="bf16 decode at batch 1 only: skip the batch-2 and batch-4 figures, the 8,192-token "
                         "prefill figures and the NVFP4 decode figures the default line also reports")
    ap.add_argument("--workload", default="decode_bf16_h2048_e128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--eager", action="store_true", help="launch every call from Python instead of HIP-graph replay")
    ap.add_argument("--separate", action="store_true",
                    help="decode: ft_moe_route then ft_moe_forward instead of the fused ft_moe_route_forward")
    ap.add_argument("--graphs", type=int, default=16, help="distinct captured steps (distinct inputs) replayed in turn")
    ap.add_argument("--tokens", type=int, default=8192, help="prefill: prompt tokens (multiples of 8192 run as chunks)")
    ap.add_argument("--act-terms", type=int, default=2, choices=(1, 2),
                    help="prefill: MXFP8 terms per activation on the matrix cores (2: within 1e-2 of the bf16 "
                         "layer; 1: half the matrix work)")
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (0 = the workload's)")
    ap.add_argument("--host-layers", type=int, default=2, help="distinct pinned host layer images (aliased)")
    ap.add_argument("--policy-study", action="store_true",
                    help="LRU workload: miss rates of expert placement policies at equal capacity (slot table only)")
    ap.add_argument("--device-fetch", action="store_true",
                    help="LRU decode: missed experts copied by ft_expert_fetch on the device (no host round trip); "
                         "the step is one captured HIP graph unless --eager")
    ap.add_argument("--coexec", action="store_true",
                    help="LRU decode: co-execution (a measured share of each layer's misses computed on the host, "
                         "the rest fetched on the device), against the graph-captured device-fetch step")
    ap.add_argument("--lookahead", action="store_true",
                    help="LRU decode routed by the routers on layer-to-layer drifting inputs: the graph-captured "
                         "step with and without look-ahead prefetch of the next layer's predicted experts")
    ap.add_argument("--ceilings", action="store_true",
                    help="only the ceiling probes (streaming read, launch floor, matrix cores, LDS-DMA), one JSON line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 256 MiB device-to-device copy (counter calibration)")
    return ap.parse_args()


def device_pool_bf16(cfg, layer, torch):
    """All expert records of one bf16 layer, generated on the device: bf16
    values of N(0, std) draws (torch's seeded generator), laid out as packed
    records."""
    from sparse_moe_expert_softmax_amd import synth
    stride = synth.record_stride(cfg.hidden, cfg.inter, cfg.w_dtype)
    assert stride == 2 * 3 * cfg.hidden * cfg.inter
    return synth.device_layer_pool(torch, cfg, layer, stride)


def ceilings(torch, reps=5):
    """Achievable ceilings on this GPU, from the probe library (libftprobe.so,
    not the MoE path): streaming reads from HBM (1 GiB, and 75 MB launches the
    size of one bf16 decode layer's expert bytes, each cold) and from the
    Infinity Cache (64 MiB read again); back-to-back empty launches; dense matrix-core
    loops (bf16, MXFP8 x MXFP4, MXFP4 x MXFP4, both instruction shapes);
    LDS-DMA from an L2-resident 2 MiB buffer (the L2 -> LDS path).  HIP events
    on the launch stream; median of reps."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_moe_expert_softmax_amd", "libftprobe.so"))
    st = torch.cuda.current_stream()
    sp = ctypes.c_void_p(st.cuda_stream)
    EV = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        fn()
        ms = []
        for _ in range(reps):
            a, b = EV(), EV()
            a.record(st)
            fn()
            b.record(st)
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return float(np.median(ms))

    def check(rc):
        if rc != 0:
            raise RuntimeError(f"probe launch failed ({rc})")

    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    sptr = ctypes.c_void_p(sink.data_ptr())
    res = {"source": "libftprobe.so (sparse_moe_expert_softmax_amd/csrc/probe.hip)"}
    def read_gbs(bufs, nbytes, passes, flags, grid):
        # median over launches, each bracketed by its own events, rotating over `bufs`
        EV = lambda: torch.cuda.Event(enable_timing=True)
        run = lambda b: check(lib.ftp_stream_read(ctypes.c_void_p(b.data_ptr()), ctypes.c_int64(nbytes),
                                                  ctypes.c_int32(passes), sptr, ctypes.c_int32(grid),
                                                  ctypes.c_int32(flags), sp))
        for b in bufs:
            run(b)
        evs = []
        for r in range(max(10, len(bufs))):
            a, z = EV(), EV()
            a.record(st)
            run(bufs[r % len(bufs)])
            z.record(st)
            evs.append((a, z))
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(z) for a, z in evs]))
        return round(nbytes * passes / (ms * 1e-3) / 1e9, 1)

    # flags: bit 0 nontemporal hint, bit 1 one contiguous range per workgroup
    rd = {}
    gib = [torch.ones(1 << 30, dtype=torch.uint8, device="cuda") for _ in range(3)]  # 3 GiB: cold in the 256 MB cache
    rd["hbm_1GiB"] = read_gbs(gib, 1 << 30, 1, 3, 8192)
    rd["hbm_1GiB_plain_loads"] = read_gbs(gib, 1 << 30, 1, 2, 8192)
    rd["hbm_1GiB_grid_stride"] = read_gbs(gib, 1 << 30, 1, 0, 8192)
    del gib
    # one decode layer's expert bytes (8 experts x 3 bf16 matrices of 2048 x 768), 40 layers rotating,
    # each launch cold: the streaming rate a launch of that size can reach
    nb = 8 * 3 * 2048 * 768 * 2
    lay = [torch.ones(nb, dtype=torch.uint8, device="cuda") for _ in range(40)]
    rd["hbm_75MB_per_launch_cold"] = read_gbs(lay, nb, 1, 3, nb // 16 // 1024)
    del lay
    mall = [torch.ones(64 << 20, dtype=torch.uint8, device="cuda")]
    rd["infinity_cache_64MiB"] = read_gbs(mall, 64 << 20, 16, 2, 8192)
    rd["infinity_cache_64MiB_grid_stride"] = read_gbs(mall, 64 << 20, 16, 0, 8192)
    del mall
    res["stream_read_gbs"] = rd
    n = 200
    ms = timed(lambda: check(lib.ftp_empty(ctypes.c_int32(n), sp)))
    res["empty_launch_us"] = round(ms * 1e3 / n, 2)
    mf = {}
    grid = 1024
    for kind, name, flop, iters, peak in ((0, "bf16_16x16x32", 16384, 4096, BF16_PEAK_TFLOPS),
                                          (3, "bf16_32x32x16", 32768, 2048, BF16_PEAK_TFLOPS),
                                          (1, "mxfp8_x_mxfp4_16x16x128", 65536, 2048, MFMA_PEAK_TFLOPS),
                                          (4, "mxfp8_x_mxfp4_32x32x64", 131072, 1024, MFMA_PEAK_TFLOPS),
                                          (2, "mxfp4_x_mxfp4_16x16x128", 65536, 2048, MXFP4_PEAK_TFLOPS),
                                          (5, "mxfp4_x_mxfp4_32x32x64", 131072, 1024, MXFP4_PEAK_TFLOPS)):
        ms = timed(lambda: check(lib.ftp_mfma(ctypes.c_int32(kind), sptr, ctypes.c_int32(grid), ctypes.c_int32(iters),
                                              sp)))
        tf = grid * 4 * iters * 8 * flop / (ms * 1e-3) / 1e12
        mf[name] = {"tflops": round(tf, 1), "frac_of_peak": round(tf / peak, 4)}
    res["mfma"] = mf
    nb, grid, iters = 2 << 20, 1024, 512
    buf = torch.ones(nb, dtype=torch.uint8, device="cuda")
    ms = timed(lambda: check(lib.ftp_lds_dma(ctypes.c_void_p(buf.data_ptr()), ctypes.c_int64(nb), sptr,
                                             ctypes.c_int32(grid), ctypes.c_int32(iters), sp)))
    moved = grid * 8 * iters * 4096
    res["lds_dma_gbs"] = round(moved / (ms * 1e-3) / 1e9, 1)
    res["lds_dma_gbs_per_cu"] = round(moved / (ms * 1e-3) / 1e9 / 256, 1)
    del buf, sink
    return res


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(cfg, batch, seconds, threads):
    """Oracle calls on fresh activations through one layer, `threads` BLAS
    threads (None = the library default), until `seconds` of timed work."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle.moe import moe_layer, route, to_f64
    from oracle.record import decode_record
    from sparse_moe_expert_softmax_amd import synth
    layer = 0
    wr = synth.router_weights(cfg, layer)
    w64 = to_f64(wr, cfg.router_dtype)
    recs = {}
    calls, tokens, t_total = 0, 0, 0.0
    wall0 = time.perf_counter()
    last = wall0
    with threadpool_limits(limits=threads):
        used = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
        while t_total < seconds and calls < 2000 and time.perf_counter() - wall0 < 4 * seconds + 60:
            x = synth.activations(cfg, 10_000 + calls, layer, batch)
            x64 = to_f64(x, cfg.act_dtype)
            ids, _, _ = route(x64, w64, cfg.top_k)
            for e in set(ids.ravel().tolist()):
                if e not in recs:
                    recs[e] = synth.expert_record(cfg, layer, e)
            t0 = time.perf_counter()
            dec = {}

            def exp_f64(e):
                if e not in dec:
                    dec[e] = decode_record(recs[e], cfg.hidden, cfg.inter, cfg.w_dtype)
                return dec[e]
            moe_layer(x64, w64, exp_f64, cfg.top_k)
            t_total += time.perf_counter() - t0
            calls += 1
            tokens += batch
            if time.perf_counter() - last > 5:
                last = time.perf_counter()
                print(f"[bench] oracle ({used} threads): {calls} calls, {t_total:.1f} s timed", file=sys.stderr,
                      flush=True)
    return tokens / t_total, calls, t_total, used


def cpu_baseline(cfg, batch, seconds):
    """fp64 oracle on a bounded sample of the same workload: fresh activations
    per call through one layer whose expert records (host generator) are made
    once and cached; generation is outside the timed region, the oracle's own
    record decoding is inside it.  Timed with the BLAS library's default
    thread count (all the cores it is allowed) and with one thread."""
    v_all, c_all, t_all, used = _oracle_rate(cfg, batch, seconds / 2, None)
    v_one, c_one, t_one, _ = _oracle_rate(cfg, batch, seconds / 2, 1)
    return {"value": v_all, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{c_all} calls of one decode layer at batch {batch} (route with exact fsum logits + "
                      f"{cfg.top_k} fp64 SwiGLU experts per token, record decoding included, generation "
                      f"excluded), {t_all:.1f} s with {used} BLAS threads (the exact router sums run on one)",
            "host_cpus": os.cpu_count(), "cpu_model": _cpu_model(),
            "one_thread": {"value": v_one, "unit": "tokens/s", "calls": c_one, "seconds": round(t_one, 1)}}


def _measure_decode_bf16(args, cfg, torch, B, pools, routers, desc, calibrate):
    """One batch size of the resident bf16 decode workload: warm-up, HIP-graph
    (or eager) timing of whole 40-layer steps, then per-call forward durations
    with the queue filled ahead; returns the figures the result line reports."""
    from sparse_moe_expert_softmax_amd import ftmoe, synth
    L, E, H, I, k = cfg.n_layers, cfg.n_experts, cfg.hidden, cfg.inter, cfg.top_k
    rec_bytes = synth.record_bytes(H, I, cfg.w_dtype)
    n_steps = args.warmup + args.steps
    xs = torch.empty((n_steps, L, B, H), dtype=torch.int16, device="cuda")
    for s in range(n_steps):
        for l in range(L):
            xs[s, l].copy_(torch.from_numpy(synth.activations(cfg, s, l, B).view(np.int16)))
    ids_all = torch.empty((n_steps, L, B, k), dtype=torch.int32, device="cuda")
    gates_all = torch.empty((n_steps, L, B, k), dtype=torch.float32, device="cuda")
    out = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(ftmoe.ft_moe_workspace_bytes(desc, B), dtype=torch.uint8, device="cuda")
    rws = torch.zeros(ftmoe.ft_route_workspace_bytes(desc, B), dtype=torch.uint8, device="cuda")
    fws = torch.zeros(ftmoe.ft_moe_route_forward_workspace_bytes(desc, B), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    print("[bench] inputs resident; warming up", file=sys.stderr, flush=True)

    def layer_call(s, l, st):
        """One MoE layer: route + forward, as one fused call unless --separate."""
        if args.separate:
            ftmoe.ft_moe_route(desc, xs[s, l], routers[l], ids_all[s, l], gates_all[s, l], workspace=rws, stream=st)
            ftmoe.ft_moe_forward(desc, xs[s, l], ids_all[s, l], gates_all[s, l], pools[l], out, ws, stream=st)
        else:
            ftmoe.ft_moe_route_forward(desc, xs[s, l], routers[l], ids_all[s, l], gates_all[s, l], pools[l], out,
                                       fws, stream=st)

    def step(s, ev=None):
        for l in range(L):
            if ev is None:
                layer_call(s, l, stream)
                continue
            # per-forward timing: the route, then the forward between events
            ftmoe.ft_moe_route(desc, xs[s, l], routers[l], ids_all[s, l], gates_all[s, l], workspace=rws,
                               stream=stream)
            ev[l][0].record(stream)
            ftmoe.ft_moe_forward(desc, xs[s, l], ids_all[s, l], gates_all[s, l], pools[l], out, ws, stream=stream)
            ev[l][1].record(stream)

    if calibrate:
        _calibration_copy(torch)
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    graphs = []
    if not args.eager:
        # one captured graph per distinct input set; replayed in turn
        n_g = min(args.graphs, args.steps)
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            for gi in range(n_g):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    step_stream = torch.cuda.current_stream()
                    for l in range(L):
                        layer_call(args.warmup + gi, l, step_stream)
                graphs.append(g)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i, s in enumerate(range(args.warmup, n_steps)):
        if graphs:
            graphs[i % len(graphs)].replay()
        else:
            step(s)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    print(f"[bench] batch {B}: timed {args.steps} steps ({'graph' if graphs else 'eager'}): {ms_per_step:.4f} ms/step",
          file=sys.stderr, flush=True)

    # per-call forward durations: HIP events on the launch stream around every
    # forward, with the queue filled ahead (a device-side sleep) so that host
    # launch latency does not fall inside the measured intervals
    n_meas = min(args.steps, 50)
    fwd_ms = []
    for s in range(args.warmup, args.warmup + n_meas):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(L)]
        torch.cuda._sleep(2_000_000)
        step(s, ev)
        torch.cuda.synchronize()
        fwd_ms.extend(a.elapsed_time(b) for a, b in ev)
    fwd_ms = np.array(fwd_ms)

    # algorithmic bytes per forward call: distinct routed experts x record bytes + x in + out
    ids_np = ids_all.cpu().numpy()
    distinct = np.array([[len(np.unique(ids_np[s, l])) for l in range(L)] for s in range(n_steps)])
    d_meas = distinct[args.warmup:args.warmup + n_meas].ravel()
    d_timed = np.array([distinct[args.warmup + (i % len(graphs) if graphs else i)].sum() for i in range(args.steps)])
    fwd_bytes = d_meas * rec_bytes + B * H * 2 + B * H * 4
    achieved_gbs = float(np.mean(fwd_bytes) / (np.mean(fwd_ms) * 1e-3) / 1e9)
    route_bytes = E * H * 2 + B * H * 2
    step_bytes = float(np.mean(d_timed)) * rec_bytes + L * (route_bytes + B * H * 4)
    layer_tok_s = B * L / (ms_per_step * 1e-3)

    return {"ms_per_step": ms_per_step, "layer_tok_s": layer_tok_s, "graphs": len(graphs), "step_bytes": step_bytes,
            "achieved_gbs": achieved_gbs, "fwd_bytes": float(np.mean(fwd_bytes)), "fwd_us": float(np.mean(fwd_ms)) * 1e3,
            "fwd_us_p10_p50_p90": [round(float(v) * 1e3, 2) for v in np.percentile(fwd_ms, [10, 50, 90])],
            "distinct": float(np.mean(d_meas))}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU: the path runs on one device, and --gpus above 1 is not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    from sparse_moe_expert_softmax_amd import ftmoe, synth
    from sparse_moe_expert_softmax_amd.configs import CONFIGS

    cfg = CONFIGS[args.workload]
    torch.cuda.set_device(0)
    if args.ceilings:
        print(json.dumps({"ceilings": ceilings(torch)}), flush=True)
        return
    if cfg.name in PREFILL_WORKLOADS:
        return run_prefill(args, cfg, torch)
    if args.policy_study:
        return run_policy_study(args, cfg, torch)
    if cfg.name == "decode_mxfp4_h4096_e256_lru" and args.lookahead:
        return run_decode_lookahead(args, cfg, torch)
    if cfg.name == "decode_mxfp4_h4096_e256_lru" and args.coexec:
        return run_decode_coexec(args, cfg, torch)
    if cfg.name == "decode_mxfp4_h4096_e256_lru":
        return run_decode_lru(args, cfg, torch)
    if cfg.name == "decode_nvfp4_h6144_e256":
        return run_decode_resident_fp4(args, cfg, torch)
    if cfg.name != "decode_bf16_h2048_e128":
        print(json.dumps({"error": f"no benchmark for workload {cfg.name}"}))
        sys.exit(2)
    B, L, E, H, I, k = args.batch, cfg.n_layers, cfg.n_experts, cfg.hidden, cfg.inter, cfg.top_k
    stride = synth.record_stride(H, I, cfg.w_dtype)
    rec_bytes = synth.record_bytes(H, I, cfg.w_dtype)
    desc = ftmoe.make_desc(cfg, stride)
    print(f"[bench] generating {L} layers x {E} experts ({L * E * stride / 1e9:.1f} GB) on the device",
          file=sys.stderr, flush=True)
    pools = [device_pool_bf16(cfg, l, torch) for l in range(L)]
    routers = [torch.from_numpy(synth.router_weights(cfg, l).view(np.int16)).cuda() for l in range(L)]
    batches = [B] + ([2, 4] if B == 1 and not args.single_batch else [])
    meas = {}
    for bq in batches:
        meas[bq] = _measure_decode_bf16(args, cfg, torch, bq, pools, routers, desc, args.calibrate_copy and bq == B)
    m = meas[B]
    ms_per_step, layer_tok_s = m["ms_per_step"], m["layer_tok_s"]
    res = {
        "metric": "moe_layer_tokens_per_s",
        "value": round(layer_tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "layers": L, "hidden": H, "experts": E, "top_k": k,
                   "inter": I, "weights": "bf16", "resident_gb": round(L * E * stride / 1e9, 1),
                   "launch": "eager" if not m["graphs"] else f"hip graphs ({m['graphs']} captured steps)",
                   "calls": "ft_moe_route + ft_moe_forward" if args.separate else "ft_moe_route_forward"},
        "stack_tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
        "step_hbm_gbs": round(m["step_bytes"] / (ms_per_step * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "kernel": "ft_moe_forward (expert GEMV)",
                     "achieved": round(m["achieved_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(m["achieved_gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": measured_decode_traffic(cfg.name, B),
                     "bytes_per_launch": round(m["fwd_bytes"]), "avg_launch_us": round(m["fwd_us"], 2),
                     "launch_us_p10_p50_p90": m["fwd_us_p10_p50_p90"],
                     "distinct_experts_per_call": round(m["distinct"], 2)},
    }
    if len(batches) > 1:  # the metric's other decode batch sizes, same layers, same process
        res["other_batches"] = {
            str(bq): {"tokens_per_s": round(meas[bq]["layer_tok_s"], 1), "ms_per_step": round(meas[bq]["ms_per_step"], 5),
                      "forward_us": round(meas[bq]["fwd_us"], 2), "forward_us_p10_p50_p90": meas[bq]["fwd_us_p10_p50_p90"],
                      "forward_bytes": round(meas[bq]["fwd_bytes"]),
                      "forward_hbm_frac": round(meas[bq]["achieved_gbs"] / HBM_PEAK_GBS, 4),
                      "distinct_experts_per_call": round(meas[bq]["distinct"], 2)} for bq in batches[1:]}
    if not args.single_batch:  # the metric's prefill half (8,192-token chunks, experts resident), NVFP4 decode
        del pools
        torch.cuda.empty_cache()
        res["prefill"] = prefill_figures(torch)
        from sparse_moe_expert_softmax_amd.configs import C6, C7
        res["prefill_bf16"] = bf16_prefill_figures(torch, C6)
        res["prefill_nvfp4"] = bf16_prefill_figures(torch, C7)
        torch.cuda.empty_cache()
        res["decode_nvfp4"] = decode_nvfp4_figures(torch)
        torch.cuda.empty_cache()
        res["ceilings"] = ceilings(torch)
        # the same forward rate against the streaming read this chip sustained in this run
        rd = res["ceilings"]["stream_read_gbs"]
        res["roofline"]["frac_of_stream_ceiling"] = round(m["achieved_gbs"] / rd["hbm_1GiB"], 4)
        res["roofline"]["frac_of_same_size_stream"] = round(m["achieved_gbs"] / rd["hbm_75MB_per_launch_cold"], 4)
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cfg, B, args.cpu_seconds)
    print(json.dumps(res), flush=True)


MFMA_PEAK_TFLOPS = 5000.0   # dense fp8 rate; the f8 x f4 instruction issues at the fp8 rate
BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix rate


def _base_result(args, metric_value, unit, ms_per_step, config, dtype):
    return {"metric": "moe_layer_tokens_per_s", "value": round(metric_value, 1), "unit": unit, "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic", "config": config}


def run_policy_study(args, cfg, torch):
    """Expert placement at equal capacity (S slots for L layers x E experts),
    on the Zipf trace and on a trace with temporal locality (each expert of a
    token kept from one step to the next with probability 0.8):
      - global LRU: one slot table for all layers (the library's);
      - per-layer split: S / L slots per layer, LRU within each (the same
        lookup kernel on one table per layer);
      - profiled static set: the S most used (layer, expert) keys over the
        first tenth of the steps stay resident, every other key is uploaded
        each time it is selected.
    Miss rates are counted over the steps after that first tenth, for every
    policy; upload bytes and host-link time follow from the record size and
    the link rate the LRU workload measures."""
    from sparse_moe_expert_softmax_amd import ftmoe, synth
    L, E, k = cfg.n_layers, cfg.n_experts, cfg.top_k
    S = cfg.n_slots
    n_steps = cfg.trace_steps
    prof = n_steps // 10
    rec = synth.record_bytes(cfg.hidden, cfg.inter, cfg.w_dtype)
    link_gbs = 54.6  # measured: ft_expert_fetch from pinned host memory
    t0 = time.perf_counter()
    traces = {"zipf": synth.zipf_trace(cfg, n_steps=n_steps, n_tokens=4),
              "sticky_p0.8": synth.sticky_trace(cfg, n_steps, 4, 0.8)}
    from sparse_moe_expert_softmax_amd import placement
    study = {}
    for tname, tr in traces.items():
        for B in (1, 4):
            ids_np = tr[:, :, :B, :].reshape(n_steps, L, B * k)
            res = {"global_lru": placement.lru_misses(torch, ids_np, E, S, per_layer=False),
                   "per_layer_lru": placement.lru_misses(torch, ids_np, E, S, per_layer=True),
                   "profiled_static": placement.profiled_static_misses(ids_np, E, S, prof)}
            distinct = placement.distinct_selected(ids_np[prof:])
            entry = {}
            for pol, m in res.items():
                if (m < 0).any():
                    raise RuntimeError(f"{pol}: slot pool exhausted")
                mm = m[prof:]
                gb = float(mm.sum(axis=1).mean() * rec / 1e9)
                entry[pol] = {"miss_rate": round(float(mm.sum() / distinct.sum()), 4),
                              "misses_per_layer_call": round(float(mm.mean()), 3),
                              "upload_gb_per_step": round(gb, 3),
                              "host_link_ms_per_step": round(gb / link_gbs * 1e3, 2)}
            study[f"{tname}_b{B}"] = entry
            print(f"[bench] policy study {tname} b={B}: " +
                  ", ".join(f"{p_} {v['miss_rate']}" for p_, v in entry.items()), file=sys.stderr, flush=True)
    wall = (time.perf_counter() - t0) * 1e3
    res = {"metric": "lru_miss_rate", "value": study["zipf_b1"]["global_lru"]["miss_rate"],
           "unit": "misses per selected expert (global LRU, Zipf trace, batch 1)", "n_gpus": 1, "steps": n_steps,
           "warmup": prof, "ms_per_step": round(wall / n_steps, 5), "higher_is_better": False, "scaling": "weak",
           "vs_baseline": None, "dtype": "int32", "data": "synthetic",
           "config": {"workload": "lru_policy_study", "layers": L, "experts": E, "top_k": k, "slots": S,
                      "record_bytes": rec, "profile_steps": prof, "link_gbs_assumed": link_gbs},
           "policies": study}
    print(json.dumps(res), flush=True)


def _layer_pool(cfg, layer, torch, stride):
    from sparse_moe_expert_softmax_amd import synth
    return synth.device_layer_pool(torch, cfg, layer, stride)


def _calibration_copy(torch):
    """One plain 256 MiB device-to-device copy: a kernel of known traffic whose
    hardware-counter readings scale the other kernels' readings."""
    src_c = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
    dst_c = torch.empty_like(src_c)
    dst_c.copy_(src_c)
    torch.cuda.synchronize()
    del src_c, dst_c


def _prefill_resident_times(torch, desc, x, routers, bufs, ids, gates, out, ws, rws, comp, n_warm, n_meas):
    """Route and forward durations (ms) of 8,192-token calls with the experts
    resident, alternating between the layer buffers and the routers; HIP
    events on the launch stream."""
    from sparse_moe_expert_softmax_amd import ftmoe
    EV = lambda: torch.cuda.Event(enable_timing=True)
    route_ms, fwd_ms = [], []
    for it in range(n_warm + n_meas):
        l = it % len(routers)
        e0, e1, e2 = EV(), EV(), EV()
        e0.record(comp)
        ftmoe.ft_moe_route(desc, x, routers[l], ids, gates, workspace=rws, stream=comp)
        e1.record(comp)
        ftmoe.ft_moe_forward(desc, x, ids, gates, bufs[it % len(bufs)], out, ws, stream=comp)
        e2.record(comp)
        if it >= n_warm:
            torch.cuda.synchronize()
            route_ms.append(e0.elapsed_time(e1))
            fwd_ms.append(e1.elapsed_time(e2))
    return np.array(route_ms), np.array(fwd_ms)


MXFP4_PEAK_TFLOPS = 10100.0  # dense MXFP4 x MXFP4 matrix rate


def prefill_figures(torch, n_meas=8):
    """The prefill half of the metric for the default line: one 8,192-token
    chunk through the 284B-like MXFP4 layer (4,096 / 2,048 / 256 experts /
    top-6) with its experts resident; two layers generated on the device,
    alternated.  Both activation modes of the matrix-core path: two MXFP8
    terms (the default, within 1e-2 of the bf16-activation layer) and one
    (half the matrix work, about 5-6% off it)."""
    from sparse_moe_expert_softmax_amd import ftmoe, synth
    from sparse_moe_expert_softmax_amd.configs import C4
    cfg, T = C4, 8192
    H, I, E, k = cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k
    stride = synth.record_stride(H, I, cfg.w_dtype)
    print("[bench] prefill figures: generating 2 MXFP4 layers on the device", file=sys.stderr, flush=True)
    bufs = [synth.device_layer_pool(torch, cfg, l, stride) for l in range(2)]
    routers = [torch.from_numpy(synth.router_weights(cfg, l).view(np.int16)).cuda() for l in range(2)]
    x = torch.from_numpy(synth.activations(cfg, 0, 0, T).view(np.int16)).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    comp = torch.cuda.current_stream()
    useful = 6.0 * T * k * H * I
    res = {"workload": cfg.name, "tokens": T, "weights": "mxfp4 resident",
           "useful_flops_per_forward": useful,
           "issued": "v_mfma_scale_f32_16x16x128_f8f6f4, MXFP8 activations x MXFP4 weights (fp8 rate)"}
    for terms in (2, 1):
        desc = ftmoe.make_desc(cfg, stride, act_terms=terms)
        ws = torch.empty(ftmoe.ft_moe_workspace_bytes(desc, T), dtype=torch.uint8, device="cuda")
        rws = torch.empty(ftmoe.ft_route_workspace_bytes(desc, T), dtype=torch.uint8, device="cuda")
        route_ms, fwd_ms = _prefill_resident_times(torch, desc, x, routers, bufs, ids, gates, out, ws, rws, comp, 2,
                                                   n_meas)
        del ws
        tflops = useful / (float(np.mean(fwd_ms)) * 1e-3) / 1e12
        t_layer = float(np.mean(route_ms + fwd_ms))
        print(f"[bench] prefill ({terms} term(s)): route {route_ms.mean():.3f} ms, forward {fwd_ms.mean():.3f} ms "
              "per layer", file=sys.stderr, flush=True)
        res["two_terms" if terms == 2 else "one_term"] = {
            "act_terms": terms, "tokens_per_s": round(T / (t_layer * 1e-3), 1),
            "route_us": round(float(route_ms.mean()) * 1e3, 1), "forward_us": round(float(fwd_ms.mean()) * 1e3, 1),
            "useful_tflops": round(tflops, 1), "issued_tflops": round(tflops * terms, 1),
            "frac_useful_of_fp8_peak": round(tflops / MFMA_PEAK_TFLOPS, 4),
            "frac_issued_of_fp8_peak": round(tflops * terms / MFMA_PEAK_TFLOPS, 4),
            "frac_useful_of_mxfp4_peak": round(tflops / MXFP4_PEAK_TFLOPS, 4),
            "traffic": measured_prefill_traffic(cfg.name, T, terms)}
    del bufs
    torch.cuda.empty_cache()
    return res


def bf16_prefill_figures(torch, cfg, n_meas=8):
    """The same for the layers on the bf16 matrix cores: one 8,192-token chunk
    through the 35B-like bf16 layer (2,048 / 768 / 128 experts / top-8) or the
    753B-like NVFP4 layer (6,144 / 2,048 / 256 / top-8) with its experts
    resident, two layers generated on the device, alternated; useful
    TFLOP/s against the dense bf16 rate."""
    from sparse_moe_expert_softmax_amd import ftmoe, synth
    from sparse_moe_expert_softmax_amd.configs import DTYPE_NAMES
    T = 8192
    H, I, k = cfg.hidden, cfg.inter, cfg.top_k
    stride = synth.record_stride(H, I, cfg.w_dtype)
    print(f"[bench] prefill figures: generating 2 {DTYPE_NAMES[cfg.w_dtype]} layers on the device", file=sys.stderr,
          flush=True)
    bufs = [synth.device_layer_pool(torch, cfg, l, stride) for l in range(2)]
    routers = [torch.from_numpy(synth.router_weights(cfg, l).view(np.int16)).cuda() for l in range(2)]
    x = torch.from_numpy(synth.activations(cfg, 0, 0, T).view(np.int16)).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    desc = ftmoe.make_desc(cfg, stride)
    ws = torch.empty(ftmoe.ft_moe_workspace_bytes(desc, T), dtype=torch.uint8, device="cuda")
    rws = torch.empty(ftmoe.ft_route_workspace_bytes(desc, T), dtype=torch.uint8, device="cuda")
    route_ms, fwd_ms = _prefill_resident_times(torch, desc, x, routers, bufs, ids, gates, out, ws, rws,
                                               torch.cuda.current_stream(), 2, n_meas)
    useful = 6.0 * T * k * H * I
    tflops = useful / (float(np.mean(fwd_ms)) * 1e-3) / 1e12
    t_layer = float(np.mean(route_ms + fwd_ms))
    print(f"[bench] prefill ({DTYPE_NAMES[cfg.w_dtype]} weights): route {route_ms.mean():.3f} ms, forward "
          f"{fwd_ms.mean():.3f} ms per layer", file=sys.stderr, flush=True)
    res = {"workload": cfg.name, "tokens": T, "weights": f"{DTYPE_NAMES[cfg.w_dtype]} resident",
           "useful_flops_per_forward": useful,
           "issued": "v_mfma_f32_16x16x32_bf16, bf16 activations x bf16 weights" +
                     (" (NVFP4 expanded exactly to bf16 in LDS)" if DTYPE_NAMES[cfg.w_dtype] == "nvfp4" else ""),
           "tokens_per_s": round(T / (t_layer * 1e-3), 1),
           "route_us": round(float(route_ms.mean()) * 1e3, 1), "forward_us": round(float(fwd_ms.mean()) * 1e3, 1),
           "useful_tflops": round(tflops, 1), "frac_of_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4),
           "traffic": measured_prefill_traffic(cfg.name, T)}
    del bufs, ws
    torch.cuda.empty_cache()
    return res


def run_prefill(args, cfg, torch):
    """8,192-token chunks through the MXFP4 or the bf16 layers: compute with
    weights resident, then the full pipeline where the next layer's whole
    expert set is copied from pinned host memory on a side stream while the
    current layer computes (two HBM layer buffers)."""
    from sparse_moe_expert_softmax_amd import ftmoe, synth
    from sparse_moe_expert_softmax_amd.configs import BF16, DTYPE_NAMES, NVFP4
    CH = 8192
    T = CH
    chunks = max(1, args.tokens // CH)
    L = args.layers or cfg.n_layers
    H, I, E, k = cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k
    stride = synth.record_stride(H, I, cfg.w_dtype)
    rec = synth.record_bytes(H, I, cfg.w_dtype)
    layer_bytes = E * stride
    bf = cfg.w_dtype in (BF16, NVFP4)   # bf16 matrix cores (NVFP4 weights expanded to bf16 on the way in)
    terms = 1 if bf else args.act_terms
    desc = ftmoe.make_desc(cfg, stride, act_terms=0 if bf else args.act_terms)
    NH = max(1, min(args.host_layers, L))
    print(f"[bench] prefill: {L} layers, {chunks} chunk(s) of {CH}; {NH} pinned host layer images "
          f"of {layer_bytes / 1e9:.2f} GB", file=sys.stderr, flush=True)
    host = []
    for h in range(NH):
        dev = _layer_pool(cfg, h, torch, stride)
        hb = torch.empty((E, stride), dtype=torch.uint8, pin_memory=True)
        hb.copy_(dev)
        host.append(hb)
        del dev
    torch.cuda.synchronize()
    bufs = [torch.empty((E, stride), dtype=torch.uint8, device="cuda") for _ in range(2)]
    for b in range(2):
        bufs[b].copy_(host[b % NH])
    routers = [torch.from_numpy(synth.router_weights(cfg, l).view(np.int16)).cuda() for l in range(L)]
    xs = [torch.from_numpy(synth.activations(cfg, c, 0, CH).view(np.int16)).cuda() for c in range(chunks)]
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(ftmoe.ft_moe_workspace_bytes(desc, T), dtype=torch.uint8, device="cuda")
    rws = torch.zeros(ftmoe.ft_route_workspace_bytes(desc, T), dtype=torch.uint8, device="cuda")
    comp = torch.cuda.current_stream()
    EV = lambda: torch.cuda.Event(enable_timing=True)
    if args.calibrate_copy:
        _calibration_copy(torch)

    # ---- compute only, weights resident (alternating the two layer buffers)
    n_warm, n_meas = max(2, args.warmup // 10), max(4, min(args.steps, L))
    route_ms, fwd_ms = _prefill_resident_times(torch, desc, xs[0], routers, bufs, ids, gates, out, ws, rws, comp,
                                               n_warm, n_meas)
    t_layer = float(np.mean(route_ms + fwd_ms))
    print(f"[bench] resident: route {route_ms.mean():.3f} ms, forward {fwd_ms.mean():.3f} ms per layer",
          file=sys.stderr, flush=True)

    # ---- one layer's upload alone: the host-link rate
    from sparse_moe_expert_softmax_amd.prefill_pipeline import PrefillPipeline
    recs_ptr = [[host[h][e].data_ptr() for e in range(E)] for h in range(NH)]
    side = torch.cuda.Stream()
    copy_ms = []
    for it in range(3):
        a, b = EV(), EV()
        a.record(side)
        ftmoe.ft_expert_upload(bufs[it % 2], stride, rec, list(range(E)), recs_ptr[it % NH], stream=side)
        b.record(side)
        torch.cuda.synchronize()
        copy_ms.append(a.elapsed_time(b))
    t_copy = float(np.median(copy_ms))
    del bufs
    torch.cuda.empty_cache()

    # ---- full pipeline (the library's double-buffered prefill): the next
    # layer's experts are copied while this layer computes
    pp = PrefillPipeline(desc, rec, compute_stream=comp)
    fws = torch.empty(ftmoe.ft_moe_route_forward_workspace_bytes(desc, T), dtype=torch.uint8, device="cuda")
    del ws
    n_total = L * chunks
    torch.cuda.synchronize()
    w0, w1 = EV(), EV()
    w0.record(comp)
    pp.start(recs_ptr[0])  # layer 0 of chunk 0: part of the pipeline fill, inside the clock
    n = 0
    for c in range(chunks):
        for l in range(L):
            nxt = recs_ptr[((n + 1) % L) % NH] if n + 1 < n_total else None
            pp.layer(nxt, xs[c], routers[l], ids, gates, out, fws)
            n += 1
    w1.record(comp)
    torch.cuda.synchronize()
    wall_ms = w0.elapsed_time(w1)
    copy_sum = t_copy * n_total
    comp_ms = t_layer * n_total
    upload_gbs = E * rec / (t_copy * 1e-3) / 1e9

    useful = 6.0 * T * k * H * I  # gate/up 4*P*H*I + down 2*P*H*I
    tflops = useful / (float(np.mean(fwd_ms)) * 1e-3) / 1e12
    peak = BF16_PEAK_TFLOPS if bf else MFMA_PEAK_TFLOPS
    res = _base_result(args, T / (t_layer * 1e-3), "tokens/s", t_layer * L,
                       {"workload": cfg.name, "tokens_per_chunk": CH, "chunks": chunks, "layers": L, "hidden": H,
                        "experts": E, "top_k": k, "inter": I, "weights": DTYPE_NAMES[cfg.w_dtype],
                        "activations": "bf16, exact on the bf16 matrix cores; h rounded to bf16" if bf else
                        f"bf16, as {terms} MXFP8 term(s) for the matrix cores",
                        "act_terms": terms}, "bf16 (f32 accumulate)" if bf else "f8xf4 (f32 accumulate)")
    res["note"] = "value = tokens/s through one MoE layer with its experts resident (route + forward)"
    res["per_layer_ms"] = {"route": round(float(route_ms.mean()), 4), "forward": round(float(fwd_ms.mean()), 4)}
    res["pipeline"] = {"wall_ms": round(wall_ms, 2), "upload_ms_sum": round(copy_sum, 2),
                       "compute_ms_sum": round(comp_ms, 2),
                       "overlap_efficiency": round(max(copy_sum, comp_ms) / wall_ms, 4),
                       "calls": "ft_prefill_pipeline_start / ft_prefill_pipeline_layer",
                       "host_link_gbs": round(upload_gbs, 2),
                       "tokens_per_s_end_to_end": round(T * chunks / (wall_ms * 1e-3), 1),
                       "host_layer_images": NH}
    res["roofline"] = {"bound": "mfma",
                       "kernel": "ft_moe_forward (grouped bf16-MFMA expert GEMM)" if bf else
                       "ft_moe_forward (grouped scaled-MFMA expert GEMM)",
                       "achieved": round(tflops, 1), "peak": peak, "unit": "TFLOP/s",
                       "frac": round(tflops / peak, 4),
                       "issued_frac": round(tflops * terms / peak, 4),
                       "traffic": measured_prefill_traffic(cfg.name, CH, terms),
                       "flops_per_launch": useful, "avg_launch_us": round(float(np.mean(fwd_ms)) * 1e3, 1)}
    print(json.dumps(res), flush=True)


def run_decode_resident_fp4(args, cfg, torch):
    """NVFP4-like decode, layers resident, batch 4, with the partition masks:
    every layer call also runs the forward on a random half of the experts and
    on the other half, and the two partial outputs must sum to the full one."""
    print(json.dumps(decode_resident_fp4(args, cfg, torch)), flush=True)


def decode_nvfp4_figures(torch):
    """The NVFP4 decode workload for the default line: 8 resident layers of the
    753B-like layer (6,144 / 2,048 / 256 experts / top-8) at 4 tokens, 30
    timed eager steps after 5, partition masks checked on the last step."""
    from sparse_moe_expert_softmax_amd.configs import C5
    a = argparse.Namespace(layers=8, batch=4, steps=30, warmup=5)
    r = decode_resident_fp4(a, C5, torch)
    rf = r["roofline"]
    return {"workload": C5.name, "batch": r["config"]["batch"], "layers": r["config"]["layers"],
            "launch": "eager", "tokens_per_s": r["value"], "ms_per_step": r["ms_per_step"],
            "forward_us": rf["avg_launch_us"], "forward_bytes": rf["bytes_per_launch"], "forward_hbm_frac": rf["frac"],
            "distinct_experts_per_call": rf["distinct_experts_per_call"],
            "partition_max_rel_err_sum_vs_full": r["partition_masks"]["max_rel_err_sum_vs_full"]}


def decode_resident_fp4(args, cfg, torch):
    from sparse_moe_expert_softmax_amd import ftmoe, synth
    L = args.layers or cfg.n_layers
    B = cfg.batches[0] if args.batch == 1 else args.batch
    H, I, E, k = cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k
    stride = synth.record_stride(H, I, cfg.w_dtype)
    rec = synth.record_bytes(H, I, cfg.w_dtype)
    desc = ftmoe.make_desc(cfg, stride)
    print(f"[bench] generating {L} NVFP4 layers ({L * E * stride / 1e9:.1f} GB) on the device", file=sys.stderr,
          flush=True)
    pools = [_layer_pool(cfg, l, torch, stride) for l in range(L)]
    routers = [torch.from_numpy(synth.router_weights(cfg, l).view(np.int16)).cuda() for l in range(L)]
    n_steps = args.warmup + args.steps
    xs = torch.stack([torch.stack([torch.from_numpy(synth.activations(cfg, s, l, B).view(np.int16))
                                   for l in range(L)]) for s in range(n_steps)]).cuda()
    masks = [torch.from_numpy(synth.partition_masks(cfg, l).view(np.int32)).cuda() for l in range(L)]
    ids = torch.empty((n_steps, L, B, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((n_steps, L, B, k), dtype=torch.float32, device="cuda")
    out = torch.empty((L, B, H), dtype=torch.float32, device="cuda")
    pa = torch.empty((B, H), dtype=torch.float32, device="cuda")
    pb = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(ftmoe.ft_moe_workspace_bytes(desc, B), dtype=torch.uint8, device="cuda")
    rws = torch.zeros(ftmoe.ft_route_workspace_bytes(desc, B), dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream()

    def step(s, ev=None):
        for l in range(L):
            ftmoe.ft_moe_route(desc, xs[s, l], routers[l], ids[s, l], gates[s, l], workspace=rws, stream=st)
            if ev is not None:
                ev[l][0].record(st)
            ftmoe.ft_moe_forward(desc, xs[s, l], ids[s, l], gates[s, l], pools[l], out[l], ws, stream=st)
            if ev is not None:
                ev[l][1].record(st)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(2_000_000)
    t0.record(st)
    for s in range(args.warmup, n_steps):
        step(s)
    t1.record(st)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    fwd_ms = []
    for s in range(args.warmup, min(n_steps, args.warmup + 20)):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(L)]
        torch.cuda._sleep(2_000_000)
        step(s, ev)
        torch.cuda.synchronize()
        fwd_ms.extend(a.elapsed_time(b) for a, b in ev)
    # partition masks: part(mask) + part(~mask) == full, on the last step
    worst = 0.0
    s = n_steps - 1
    for l in range(L):
        ftmoe.ft_moe_forward(desc, xs[s, l], ids[s, l], gates[s, l], pools[l], out[l], ws, stream=st)
        full = out[l].clone()
        for m in masks[l]:
            comp_m = (~m).contiguous()
            ftmoe.ft_moe_forward(desc, xs[s, l], ids[s, l], gates[s, l], pools[l], pa, ws, expert_mask=m, stream=st)
            ftmoe.ft_moe_forward(desc, xs[s, l], ids[s, l], gates[s, l], pools[l], pb, ws, expert_mask=comp_m,
                                 stream=st)
            worst = max(worst, float(((pa + pb) - full).abs().max() / full.abs().max()))
    ids_np = ids.cpu().numpy()
    distinct = np.array([[len(np.unique(ids_np[s_, l])) for l in range(L)]
                         for s_ in range(args.warmup, min(n_steps, args.warmup + 20))]).ravel()
    fwd_bytes = distinct * rec + B * H * 2 + B * H * 4
    gbs = float(np.mean(fwd_bytes) / (np.mean(fwd_ms) * 1e-3) / 1e9)
    res = _base_result(args, B * L / (ms_per_step * 1e-3), "tokens/s", ms_per_step,
                       {"workload": cfg.name, "batch": B, "layers": L, "hidden": H, "experts": E, "top_k": k,
                        "inter": I, "weights": "nvfp4-like (e2m1, e4m3 per 16, fp32 per tensor)",
                        "resident_gb": round(L * E * stride / 1e9, 1), "launch": "eager"}, "bf16")
    res["partition_masks"] = {"masks_per_layer": int(masks[0].shape[0]), "max_rel_err_sum_vs_full": worst}
    res["roofline"] = {"bound": "hbm", "kernel": "ft_moe_forward (expert GEMV)", "achieved": round(gbs, 1),
                       "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                       "bytes_per_launch": round(float(np.mean(fwd_bytes))),
                       "avg_launch_us": round(float(np.mean(fwd_ms)) * 1e3, 2),
                       "distinct_experts_per_call": round(float(np.mean(distinct)), 2)}
    return res


def run_decode_lru(args, cfg, torch):
    """MXFP4 decode through the global LRU slot pool, routing driven by the
    seeded Zipf trace (selection bias), cold start; misses are uploaded from
    pinned host memory on a side stream before the layer's forward."""
    from sparse_moe_expert_softmax_amd import ftmoe, synth
    L = args.layers or cfg.n_layers
    B = args.batch
    H, I, E, k = cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k
    S = int(cfg.pool_fraction * E * L)
    stride = synth.record_stride(H, I, cfg.w_dtype)
    rec = synth.record_bytes(H, I, cfg.w_dtype)
    desc = ftmoe.make_desc(cfg, stride)
    NH = max(1, min(args.host_layers, L))
    n_steps = min(cfg.trace_steps, args.warmup + args.steps)
    print(f"[bench] LRU decode: {L} layers, pool {S} slots ({S * stride / 1e9:.1f} GB), {NH} pinned host layer "
          f"images, {n_steps} trace steps at batch {B}", file=sys.stderr, flush=True)
    host = []
    for h in range(NH):
        dev = _layer_pool(cfg, h, torch, stride)
        hb = torch.empty((E, stride), dtype=torch.uint8, pin_memory=True)
        hb.copy_(dev)
        host.append(hb)
        del dev
    host_ptr = [[host[h][e].data_ptr() for e in range(E)] for h in range(NH)]
    pool = torch.empty((S, stride), dtype=torch.uint8, device="cuda")
    table = torch.zeros(ftmoe.ft_slot_table_bytes(L, E, S), dtype=torch.uint8, device="cuda")
    ftmoe.ft_slot_table_init(table, L, E, S)
    trace = synth.zipf_trace(cfg, n_steps=n_steps)
    routers = [torch.from_numpy(synth.router_weights(cfg, l).view(np.int16)).cuda() for l in range(L)]
    g = torch.Generator(device="cuda")
    g.manual_seed(synth.ENTROPY + 3)
    ids = torch.empty((B, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((B, k), dtype=torch.float32, device="cuda")
    slots = torch.empty((B, k), dtype=torch.int32, device="cuda")
    flags = torch.empty((B, k), dtype=torch.uint8, device="cuda")
    mlist = torch.empty(2 * B * k + 1, dtype=torch.int32, device="cuda")  # [n_miss, (e, slot)...]
    h_mlist = torch.empty(2 * B * k + 1, dtype=torch.int32, pin_memory=True)
    bias = torch.zeros((B, E), dtype=torch.float32, device="cuda")
    out = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(ftmoe.ft_moe_workspace_bytes(desc, B), dtype=torch.uint8, device="cuda")
    rws = torch.zeros(ftmoe.ft_route_workspace_bytes(desc, B), dtype=torch.uint8, device="cuda")
    comp = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    trace_dev = torch.from_numpy(trace[:, :, :B, :].astype(np.int64)).cuda()
    EV = lambda: torch.cuda.Event(enable_timing=True)
    misses, step_ms, fwd_ms, up_ev = [], [], [], []
    import time as _t
    xs = torch.randn((64, B, H), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    if args.device_fetch:  # the layer's host record addresses, on the device; miss counts stay there too
        src_dev = [torch.tensor(host_ptr[h], dtype=torch.int64, device="cuda") for h in range(NH)]
        nm_dev = torch.zeros(n_steps * L, dtype=torch.int32, device="cuda")
        fetch_ev = []
    fstep = None
    if args.device_fetch and not args.eager:
        # the whole step (route, lookup, fetch, forward per layer) as one HIP
        # graph; each step's activations and trace bias are staged into its
        # fixed input buffers first
        from sparse_moe_expert_softmax_amd.decode_step import DeviceFetchStep
        fstep = DeviceFetchStep(desc, L, B, table, S, pool, rec, routers, [src_dev[l % NH] for l in range(L)])
        fstep.capture()
        torch.cuda.synchronize()
        x_idx = [torch.tensor([(s_ * L + l) % 64 for l in range(L)], device="cuda") for s_ in range(n_steps)]
    for s_ in range(n_steps):
        if fstep is not None:
            t_s = _t.perf_counter()
            torch.index_select(xs, 0, x_idx[s_], out=fstep.x)
            fstep.bias.zero_()
            fstep.bias.scatter_(2, trace_dev[s_], 30.0)
            fstep.run()
            nm_dev[s_ * L:(s_ + 1) * L].copy_(fstep.mlist[:, 0])
            comp.synchronize()
            if s_ >= args.warmup:
                step_ms.append((_t.perf_counter() - t_s) * 1e3)
            continue
        t_s = _t.perf_counter()
        for l in range(L):
            x = xs[(s_ * L + l) % 64]
            bias.zero_()
            bias.scatter_(1, trace_dev[s_, l], 30.0)
            ftmoe.ft_moe_route(desc, x, routers[l], ids, gates, sel_bias=bias, workspace=rws, stream=comp)
            ftmoe.ft_slot_lookup(table, l, ids, slots, flags, mlist[1:], mlist[:1], stream=comp)
            if args.device_fetch:
                a, b = EV(), EV()
                a.record(comp)
                ftmoe.ft_expert_fetch(pool, stride, rec, E, S, src_dev[l % NH], mlist[1:], mlist[:1], B * k,
                                      stream=comp)
                b.record(comp)
                nm_dev[s_ * L + l].copy_(mlist[0])
                if s_ >= args.warmup:
                    fetch_ev.append((a, b, s_ * L + l))
                e0, e1 = EV(), EV()
                e0.record(comp)
                ftmoe.ft_moe_forward(desc, x, ids, gates, pool, out, ws, slot_ids=slots, stream=comp)
                e1.record(comp)
                if s_ >= args.warmup:
                    fwd_ms.append((e0, e1))
                continue
            h_mlist.copy_(mlist, non_blocking=True)
            comp.synchronize()
            nm = int(h_mlist[0])
            if nm < 0:
                raise RuntimeError("slot pool exhausted")
            if nm:
                pairs = h_mlist[1:1 + 2 * nm].tolist()
                es, ss = pairs[0::2], pairs[1::2]
                a, b, done = EV(), EV(), torch.cuda.Event()
                a.record(side)
                ftmoe.ft_expert_upload(pool, stride, rec, ss, [host_ptr[l % NH][e] for e in es], stream=side,
                                       done_event=done)
                b.record(side)
                comp.wait_event(done)
                if s_ >= args.warmup:
                    up_ev.append((a, b, nm))
            e0, e1 = EV(), EV()
            e0.record(comp)
            ftmoe.ft_moe_forward(desc, x, ids, gates, pool, out, ws, slot_ids=slots, stream=comp)
            e1.record(comp)
            if s_ >= args.warmup:
                fwd_ms.append((e0, e1))
            misses.append(nm)
        comp.synchronize()
        if s_ >= args.warmup:
            step_ms.append((_t.perf_counter() - t_s) * 1e3)
    torch.cuda.synchronize()
    if args.device_fetch:
        misses = nm_dev.cpu().tolist()
        if min(misses) < 0:
            raise RuntimeError("slot pool exhausted")
        up_ev = [(a, b, misses[i]) for a, b, i in fetch_ev]
    # records copied in the timed steps (fetch durations only exist when launched eagerly)
    n_up = (sum(misses[args.warmup * L:]) if fstep is not None else sum(n for _, _, n in up_ev))
    # kernel-level forward time without host gaps: replay recorded calls with the queue filled ahead
    rec_calls = []
    for s_ in range(max(args.warmup, n_steps - 4), n_steps):
        for l in range(L):
            bias.zero_()
            bias.scatter_(1, trace_dev[s_, l], 30.0)
            i_ = torch.empty_like(ids); g_ = torch.empty_like(gates)
            ftmoe.ft_moe_route(desc, xs[(s_ * L + l) % 64], routers[l], i_, g_, sel_bias=bias, workspace=rws,
                               stream=comp)
            ftmoe.ft_slot_lookup(table, l, i_, slots, flags, mlist[1:], mlist[:1], stream=comp)
            rec_calls.append((xs[(s_ * L + l) % 64], i_, g_, slots.clone()))
    torch.cuda.synchronize()
    f_res = []
    torch.cuda._sleep(2_000_000)
    for x_, i_, g_, sl_ in rec_calls:
        e0, e1 = EV(), EV()
        e0.record(comp)
        ftmoe.ft_moe_forward(desc, x_, i_, g_, pool, out, ws, slot_ids=sl_, stream=comp)
        e1.record(comp)
        f_res.append((e0, e1))
    torch.cuda.synchronize()
    f_res_ms = np.array([a.elapsed_time(b) for a, b in f_res])
    d_res = np.array([len(np.unique(i_.cpu().numpy())) for _, i_, _, _ in rec_calls])
    up_ms = sum(a.elapsed_time(b) for a, b, _ in up_ev)
    f_ms = np.array([a.elapsed_time(b) for a, b in fwd_ms]) if fwd_ms else None
    miss_arr = np.array(misses).reshape(n_steps, L)
    # distinct experts per call = the trace's distinct ids (routing follows the trace)
    distinct = np.array([[len(np.unique(trace[s_, l, :B])) for l in range(L)] for s_ in range(args.warmup, n_steps)])
    fwd_bytes = d_res * rec + B * H * 2 + B * H * 4
    gbs = float(np.mean(fwd_bytes) / (np.mean(f_res_ms) * 1e-3) / 1e9)
    t_step = float(np.mean(step_ms))
    res = _base_result(args, B * L / (t_step * 1e-3), "tokens/s", t_step,
                       {"workload": cfg.name, "batch": B, "layers": L, "hidden": H, "experts": E, "top_k": k,
                        "inter": I, "weights": "mxfp4", "pool_slots": S, "pool_gb": round(S * stride / 1e9, 1),
                        "trace": f"zipf s={cfg.zipf_s}, {n_steps} steps, cold start", "host_layer_images": NH,
                        "launch": ("one HIP graph per step: route, lookup, on-device fetch, forward per layer"
                                   if fstep is not None else
                                   "eager, misses fetched on the device (ft_expert_fetch, no host round trip)"
                                   if args.device_fetch else
                                   "eager, host-synchronous per layer (miss list read back before uploads)")},
                       "bf16")
    res["steps"] = n_steps - args.warmup
    res["lru"] = {"miss_rate_per_selected_expert": round(float(miss_arr[args.warmup:].sum() / distinct.sum()), 4),
                  "misses_per_layer_call": round(float(miss_arr[args.warmup:].mean()), 3),
                  "cold_start_misses_first_step": int(miss_arr[0].sum()),
                  "upload_gb_per_step": round(float(n_up * rec / max(1, len(step_ms)) / 1e9), 3),
                  "host_link_gbs": round(n_up * rec / (up_ms * 1e-3) / 1e9, 2) if up_ms > 0 else None}
    res["roofline"] = {"bound": "hbm", "kernel": "ft_moe_forward (expert GEMV, slot-indirected)",
                       "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                       "bytes_per_launch": round(float(np.mean(fwd_bytes))),
                       "avg_launch_us": round(float(np.mean(f_res_ms)) * 1e3, 2),
                       "note": "forward calls of the last trace steps replayed with the queue filled ahead"
                               + ("" if f_ms is None else "; in the timed loop the forward averaged "
                                  f"{float(np.mean(f_ms)) * 1e3:.1f} us")}
    print(json.dumps(res), flush=True)


def run_decode_coexec(args, cfg, torch):
    """MXFP4 decode through the global LRU pool on the Zipf trace, twice on
    the same trace and inputs from a cold start: (1) co-execution (CoExecStep:
    per layer, a measured share q of the misses computed on the host CPU, the
    rest fetched on the device), (2) the graph-captured device-fetch step
    (every miss fetched).  Step times, miss split and host-leg time."""
    from sparse_moe_expert_softmax_amd import ftmoe, synth
    from sparse_moe_expert_softmax_amd.coexec import CoExecStep
    from sparse_moe_expert_softmax_amd.decode_step import DeviceFetchStep
    L = args.layers or cfg.n_layers
    B = args.batch
    H, I, E, k = cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k
    S = int(cfg.pool_fraction * E * L)
    stride = synth.record_stride(H, I, cfg.w_dtype)
    rec = synth.record_bytes(H, I, cfg.w_dtype)
    desc = ftmoe.make_desc(cfg, stride)
    NH = max(1, min(args.host_layers, L))
    n_steps = min(cfg.trace_steps, args.warmup + args.steps)
    print(f"[bench] co-execution: {L} layers, pool {S} slots, {n_steps} trace steps at batch {B}", file=sys.stderr,
          flush=True)
    host = []
    for h in range(NH):
        d_ = _layer_pool(cfg, h, torch, stride)
        hb = torch.empty((E, stride), dtype=torch.uint8, pin_memory=True)
        hb.copy_(d_)
        host.append(hb)
        del d_
    host_ptr = [[host[h][e].data_ptr() for e in range(E)] for h in range(NH)]
    src_dev = [torch.tensor(host_ptr[h], dtype=torch.int64, device="cuda") for h in range(NH)]
    routers = [torch.from_numpy(synth.router_weights(cfg, l).view(np.int16)).cuda() for l in range(L)]
    trace = synth.zipf_trace(cfg, n_steps=n_steps)
    trace_dev = torch.from_numpy(trace[:, :, :B, :].astype(np.int64)).cuda()
    g = torch.Generator(device="cuda")
    g.manual_seed(synth.ENTROPY + 3)
    xs = torch.randn((64, B, H), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    x_idx = [torch.tensor([(s_ * L + l) % 64 for l in range(L)], device="cuda") for s_ in range(n_steps)]
    results = {}
    for mode in ("coexec", "device_fetch"):
        pool = torch.empty((S, stride), dtype=torch.uint8, device="cuda")
        table = torch.zeros(ftmoe.ft_slot_table_bytes(L, E, S), dtype=torch.uint8, device="cuda")
        ftmoe.ft_slot_table_init(table, L, E, S)
        x = torch.empty((L, B, H), dtype=torch.bfloat16, device="cuda")
        bias = torch.zeros((L, B, E), dtype=torch.float32, device="cuda")
        if mode == "coexec":
            st = CoExecStep(desc, L, B, table, S, pool, rec, routers, [src_dev[l % NH] for l in range(L)],
                            [host_ptr[l % NH] for l in range(L)])
            cal = st.calibrate()
            print(f"[bench] calibration: link {cal['link_gbs']:.1f} GB/s, host {cal['host_gbs']:.1f} GB/s, "
                  f"q = {cal['q']:.3f}", file=sys.stderr, flush=True)
        else:
            st = DeviceFetchStep(desc, L, B, table, S, pool, rec, routers, [src_dev[l % NH] for l in range(L)])
            st.capture()
        torch.cuda.synchronize()
        step_ms, host_ms, n_host, n_up = [], [], 0, 0
        for s_ in range(n_steps):
            t0 = time.perf_counter()
            if mode == "coexec":
                torch.index_select(xs, 0, x_idx[s_], out=x)
                bias.zero_()
                bias.scatter_(2, trace_dev[s_], 30.0)
                st.step(x, bias)
            else:
                torch.index_select(xs, 0, x_idx[s_], out=st.x)
                st.bias.zero_()
                st.bias.scatter_(2, trace_dev[s_], 30.0)
                st.run()
            torch.cuda.current_stream().synchronize()
            if s_ >= args.warmup:
                step_ms.append((time.perf_counter() - t0) * 1e3)
                if mode == "coexec":
                    host_ms.append(st.host_ms)
                    n_host += sum(len(c) for c in st.host_sets)
                    n_up += sum(len(u) for u in st.uploaded)
                else:
                    n_up += int(st.mlist[:, 0].sum())
        nt = len(step_ms)
        r = {"ms_per_step": round(float(np.mean(step_ms)), 3), "tokens_per_s": round(B * L / (np.mean(step_ms) * 1e-3), 1),
             "uploaded_per_step": round(n_up / nt, 2), "host_computed_per_step": round(n_host / nt, 2)}
        if mode == "coexec":
            r.update({"q": round(cal["q"], 4), "link_gbs": round(cal["link_gbs"], 1),
                      "host_gbs": round(cal["host_gbs"], 1), "host_leg_ms_per_step": round(float(np.mean(host_ms)), 3)})
        results[mode] = r
        print(f"[bench] {mode}: {r}", file=sys.stderr, flush=True)
        del st, pool, table
        torch.cuda.empty_cache()
    c, f = results["coexec"], results["device_fetch"]
    res = _base_result(args, c["tokens_per_s"], "tokens/s", c["ms_per_step"],
                       {"workload": cfg.name, "batch": B, "layers": L, "experts": E, "top_k": k, "slots": S,
                        "trace": f"zipf s={cfg.zipf_s}, {n_steps} steps, cold start", "host_layer_images": NH,
                        "calls": "route, ft_slot_probe, host split, ft_slot_lookup, ft_expert_fetch, ft_moe_forward "
                                 "(mask), ft_moe_forward_host, ft_moe_add_partial per layer"}, "bf16")
    res["steps"] = n_steps - args.warmup
    res["coexec"] = c
    res["device_fetch_graph"] = f
    res["speedup_vs_device_fetch"] = round(f["ms_per_step"] / c["ms_per_step"], 4)
    print(json.dumps(res), flush=True)


def run_decode_lookahead(args, cfg, torch):
    """MXFP4 decode through the global LRU pool (43 layers, 2,752 slots), routed
    by the layers' own routers on inputs that drift from layer to layer with
    correlation alpha (synth.layer_correlated_activations), batch B.  For
    each alpha, the graph-captured step without and with look-ahead prefetch
    (the next layer's router on this layer's input predicts its experts,
    which are copied on a side stream while this layer computes), each from
    a cold cache: step time, misses of the real lookups, predicted experts
    copied and the share of them the next layer used."""
    from sparse_moe_expert_softmax_amd import ftmoe, synth
    from sparse_moe_expert_softmax_amd.lookahead import LookaheadStep
    L = args.layers or cfg.n_layers
    B = args.batch
    H, I, E, k = cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k
    S = int(cfg.pool_fraction * E * L)
    stride = synth.record_stride(H, I, cfg.w_dtype)
    rec = synth.record_bytes(H, I, cfg.w_dtype)
    desc = ftmoe.make_desc(cfg, stride)
    NH = max(1, min(args.host_layers, L))
    n_steps = args.warmup + args.steps
    host = []
    for h in range(NH):
        d_ = _layer_pool(cfg, h, torch, stride)
        hb = torch.empty((E, stride), dtype=torch.uint8, pin_memory=True)
        hb.copy_(d_)
        host.append(hb)
        del d_
    src_dev = [torch.tensor([host[h][e].data_ptr() for e in range(E)], dtype=torch.int64, device="cuda")
               for h in range(NH)]
    routers = [torch.from_numpy(synth.router_weights(cfg, l).view(np.int16)).cuda() for l in range(L)]
    results = {}
    for alpha in (0.0, 0.9, 0.99):
        xs = [torch.from_numpy(synth.layer_correlated_activations(cfg, s_, B, alpha).view(np.int16)).cuda()
              for s_ in range(n_steps)]
        for la in (False, True):
            pool = torch.empty((S, stride), dtype=torch.uint8, device="cuda")
            table = torch.zeros(ftmoe.ft_slot_table_bytes(L, E, S), dtype=torch.uint8, device="cuda")
            ftmoe.ft_slot_table_init(table, L, E, S)
            st = LookaheadStep(desc, L, B, table, S, pool, rec, routers, [src_dev[l % NH] for l in range(L)],
                               lookahead=la)
            st.capture()
            torch.cuda.synchronize()
            step_ms, miss, pmiss, used, pred = [], 0, 0, 0, 0
            for s_ in range(n_steps):
                st.x.view(torch.int16).copy_(xs[s_])
                t0 = time.perf_counter()
                st.run()
                torch.cuda.current_stream().synchronize()
                if s_ >= args.warmup:
                    step_ms.append((time.perf_counter() - t0) * 1e3)
                    miss += int(st.mlist[:, 0].sum())
                    if la:
                        pmiss += int(st.pmlist[1:, 0].sum())
                        ids = st.ids.cpu().numpy()
                        pr = st.pred_ids.cpu().numpy()
                        for l in range(1, L):
                            p_ = set(pr[l].ravel().tolist())
                            used += len(p_ & set(ids[l].ravel().tolist()))
                            pred += len(p_)
            nt = len(step_ms)
            r = {"ms_per_step": round(float(np.mean(step_ms)), 3),
                 "tokens_per_s": round(B * L / (np.mean(step_ms) * 1e-3), 1),
                 "real_misses_per_step": round(miss / nt, 2)}
            if la:
                r.update({"prefetched_per_step": round(pmiss / nt, 2),
                          "predicted_used_share": round(used / max(pred, 1), 4)})
            results[f"alpha_{alpha}_{'lookahead' if la else 'plain'}"] = r
            print(f"[bench] alpha {alpha} lookahead={la}: {r}", file=sys.stderr, flush=True)
            del st, pool, table
            torch.cuda.empty_cache()
    main_r = results["alpha_0.9_lookahead"]
    res = _base_result(args, main_r["tokens_per_s"], "tokens/s", main_r["ms_per_step"],
                       {"workload": cfg.name + "_routed_drift", "batch": B, "layers": L, "experts": E, "top_k": k,
                        "slots": S, "inputs": "layer-to-layer correlation alpha (0, 0.9, 0.99), routed by the "
                                              "layers' routers", "host_layer_images": NH,
                        "launch": "one HIP graph per step (two streams with look-ahead)"}, "bf16")
    res["lookahead"] = results
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
