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
the forward's measured duration, against the 8 TB/s HBM peak), and the fp64
oracle timed on this host's cores on a bounded sample of the same workload.
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--workload", default="decode_bf16_h2048_e128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--eager", action="store_true", help="launch every call from Python instead of HIP-graph replay")
    ap.add_argument("--graphs", type=int, default=16, help="distinct captured steps (distinct inputs) replayed in turn")
    return ap.parse_args()


def device_pool_bf16(cfg, layer, torch):
    """All expert records of one layer, generated on the device: bf16 values of
    N(0, std) draws (torch's seeded generator), laid out as packed records."""
    from sparse_moe_expert_softmax_amd import synth
    stride = synth.record_stride(cfg.hidden, cfg.inter, cfg.w_dtype)
    n = 3 * cfg.hidden * cfg.inter
    assert stride == 2 * n
    g = torch.Generator(device="cuda")
    g.manual_seed(synth.ENTROPY * 1000 + cfg.cid * 100 + layer)
    w = torch.empty((cfg.n_experts, n), dtype=torch.bfloat16, device="cuda")
    for e in range(cfg.n_experts):
        w[e].copy_(torch.randn(n, generator=g, device="cuda", dtype=torch.float32).mul_(cfg.weight_std))
    return w.view(torch.uint8).view(cfg.n_experts, stride)


def cpu_baseline(cfg, batch, seconds):
    """fp64 oracle on a bounded sample of the same workload (host generator)."""
    from threadpoolctl import threadpool_limits

    from oracle.moe import moe_layer, to_f64
    from oracle.record import decode_record
    from sparse_moe_expert_softmax_amd import synth
    calls, tokens = 0, 0
    t_total = 0.0
    with threadpool_limits(limits=1):
        layer = 0
        while t_total < seconds and calls < 1000:
            x = synth.activations(cfg, 10_000 + calls, layer, batch)
            wr = synth.router_weights(cfg, layer)
            recs = {}

            def expert(e):
                if e not in recs:
                    recs[e] = synth.expert_record(cfg, layer, e)
                return recs[e]
            # generation is excluded from the timing: pre-generate the records routed
            from oracle.moe import route
            ids, _, _ = route(to_f64(x, cfg.act_dtype), to_f64(wr, cfg.router_dtype), cfg.top_k)
            for e in set(ids.ravel().tolist()):
                expert(e)
            t0 = time.perf_counter()
            dec = {}

            def exp_f64(e):
                if e not in dec:
                    dec[e] = decode_record(recs[e], cfg.hidden, cfg.inter, cfg.w_dtype)
                return dec[e]
            moe_layer(to_f64(x, cfg.act_dtype), to_f64(wr, cfg.router_dtype), exp_f64, cfg.top_k)
            t_total += time.perf_counter() - t0
            calls += 1
            tokens += batch
            layer = (layer + 1) % cfg.n_layers
    return {"value": tokens / t_total, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{calls} layer calls of the same decode layer at batch {batch} "
                      f"(route + {cfg.top_k} experts per token, fp64, expert decode included, "
                      f"generation excluded), {t_total:.1f} s on 1 thread"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU; multi-GPU runs are not part of it",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    from sparse_moe_expert_softmax_amd import ftmoe, synth
    from sparse_moe_expert_softmax_amd.configs import CONFIGS

    cfg = CONFIGS[args.workload]
    if cfg.name != "decode_bf16_h2048_e128":
        print(json.dumps({"error": f"workload {cfg.name} is run by bench_workloads.py"}))
        sys.exit(2)
    torch.cuda.set_device(0)
    B, L, E, H, I, k = args.batch, cfg.n_layers, cfg.n_experts, cfg.hidden, cfg.inter, cfg.top_k
    stride = synth.record_stride(H, I, cfg.w_dtype)
    rec_bytes = synth.record_bytes(H, I, cfg.w_dtype)
    desc = ftmoe.make_desc(cfg, stride)
    print(f"[bench] generating {L} layers x {E} experts ({L * E * stride / 1e9:.1f} GB) on the device",
          file=sys.stderr, flush=True)
    pools = [device_pool_bf16(cfg, l, torch) for l in range(L)]
    routers = [torch.from_numpy(synth.router_weights(cfg, l).view(np.int16)).cuda() for l in range(L)]
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
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    print("[bench] inputs resident; warming up", file=sys.stderr, flush=True)

    def step(s, ev=None):
        for l in range(L):
            ftmoe.ft_moe_route(desc, xs[s, l], routers[l], ids_all[s, l], gates_all[s, l], workspace=rws,
                               stream=stream)
            if ev is not None:
                ev[l][0].record(stream)
            ftmoe.ft_moe_forward(desc, xs[s, l], ids_all[s, l], gates_all[s, l], pools[l], out, ws, stream=stream)
            if ev is not None:
                ev[l][1].record(stream)

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
                        s_ = args.warmup + gi
                        ftmoe.ft_moe_route(desc, xs[s_, l], routers[l], ids_all[s_, l], gates_all[s_, l],
                                           workspace=rws, stream=step_stream)
                        ftmoe.ft_moe_forward(desc, xs[s_, l], ids_all[s_, l], gates_all[s_, l], pools[l], out, ws,
                                             stream=step_stream)
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
    print(f"[bench] timed {args.steps} steps ({'graph' if graphs else 'eager'}): {ms_per_step:.4f} ms/step",
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
                   "launch": "eager" if not graphs else f"hip graphs ({len(graphs)} captured steps)"},
        "stack_tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
        "step_hbm_gbs": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "kernel": "ft_moe_forward (expert GEMV)",
                     "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": round(float(np.mean(fwd_bytes))), "avg_launch_us": round(float(np.mean(fwd_ms)) * 1e3, 2),
                     "distinct_experts_per_call": round(float(np.mean(d_meas)), 2)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cfg, B, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
