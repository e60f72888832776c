"""One decode step through the global expert cache with co-execution: a
share of each layer's missed experts is computed on the host CPU instead of
being copied to the device.

The pages split a decode step's cache misses between a transfer over the
host link (the expert is then computed, and cached, on the device) and
computation in place on the host CPU, with the split ratio taken from the
machine's measured bandwidths; both run at once and the partial outputs are
summed, which keeps the MoE output exact (FreeToken explainer page, "how"
section, decode passage; architecture guide, decode passage).

Per layer, on one stream: route; residency probe of the selected ids; one
host synchronisation to read the ids, gates and residency; the host picks
the set C of missed experts it will compute (round(q * misses) of them:
those selected least often so far, so that
rarely used experts are computed in place and do not displace frequently
used ones from the cache); the lookup runs on the ids with C's entries set
to -1 (so C takes no slot and evicts nothing); the device copies the
remaining misses from pinned host memory (ft_expert_fetch) and runs the
forward on every selected expert except C (mask); meanwhile the host runs
ft_moe_forward_host on C from the same pinned records; its partial output
is copied over and added (ft_moe_add_partial).

q is the host's share of the combined rate: q = B_host / (B_host + B_link),
with B_link the measured device-side copy rate of records from pinned host
memory and B_host the measured rate at which ft_moe_forward_host consumes
record bytes (`calibrate`).

This is argument plumbing around the C entry points: every step of the
layer runs in the library (device kernels, or its host leg)."""
import time

import numpy as np
import torch

from . import ftmoe


def _bitset(ids, n_experts):
    m = np.zeros((n_experts + 31) // 32, dtype=np.uint32)
    for e in ids:
        m[e >> 5] |= np.uint32(1 << (e & 31))
    return m


class CoExecStep:
    """Buffers and the per-layer sequence of one co-executed decode step over
    `n_layers` layers at `n_tokens` tokens.

    routers[l]: device router weights; layer_src_dev[l]: device int64 tensor
    of layer l's pinned host record addresses; layer_src_host[l]: the same
    addresses as a Python list.  Inputs per step: x [L, T, H] (device, the
    descriptor's act dtype) and optionally bias [L, T, E] (device fp32,
    selection only).  Outputs after `step`: out [L, T, H] (device), ids,
    gates, slots (device), and host_sets[l] / uploaded[l] (host lists)."""

    def __init__(self, desc, n_layers, n_tokens, table, n_slots, pool, record_bytes, routers, layer_src_dev,
                 layer_src_host, q=None, n_threads=0):
        H, E, k = desc.hidden, desc.n_experts, desc.top_k
        L, T = n_layers, n_tokens
        if len(routers) != L or len(layer_src_dev) != L or len(layer_src_host) != L:
            raise ValueError("one router and one host address table per layer")
        self.desc, self.L, self.T = desc, L, T
        self.table, self.pool, self.rec, self.n_slots = table, pool, record_bytes, n_slots
        # the device-side copy moves 16-byte pieces: round the record up (the
        # padding up to the stride exists in the host records and the pool)
        self.fetch_bytes = (record_bytes + 15) // 16 * 16
        if self.fetch_bytes > desc.expert_stride:
            raise ValueError("record bytes rounded to 16 exceed the expert stride")
        self.routers, self.src_dev, self.src_host = routers, layer_src_dev, layer_src_host
        self.q, self.n_threads = q, n_threads
        dev = pool.device
        self.ids = torch.empty((L, T, k), dtype=torch.int32, device=dev)
        self.ids_lk = torch.empty((L, T, k), dtype=torch.int32, device=dev)
        self.gates = torch.empty((L, T, k), dtype=torch.float32, device=dev)
        self.slots = torch.empty((L, T, k), dtype=torch.int32, device=dev)
        self.flags = torch.empty((L, T, k), dtype=torch.uint8, device=dev)
        self.res = torch.empty((L, T, k), dtype=torch.uint8, device=dev)
        self.mlist = torch.empty((L, 2 * T * k + 1), dtype=torch.int32, device=dev)
        self.mask = torch.empty((L, (E + 31) // 32), dtype=torch.int32, device=dev)
        self.out = torch.empty((L, T, H), dtype=torch.float32, device=dev)
        self.part = torch.empty((T, H), dtype=torch.float32, device=dev)
        self.ws = torch.empty(max(ftmoe.ft_moe_workspace_bytes(desc, T), 256), dtype=torch.uint8, device=dev)
        self.rws = torch.empty(max(ftmoe.ft_route_workspace_bytes(desc, T), 256), dtype=torch.uint8, device=dev)
        # pinned host staging (every write to it follows a synchronisation that
        # covers the copies that read it before)
        self.h_ids = torch.empty((T, k), dtype=torch.int32, pin_memory=True)
        self.h_gates = torch.empty((T, k), dtype=torch.float32, pin_memory=True)
        self.h_res = torch.empty((T, k), dtype=torch.uint8, pin_memory=True)
        self.h_x = torch.empty((T, H), dtype=torch.int16 if desc.act_dtype == 1 else torch.float32, pin_memory=True)
        self.h_lk = torch.empty((L, T, k), dtype=torch.int32, pin_memory=True)
        self.h_mask = torch.empty((L, (E + 31) // 32), dtype=torch.int32, pin_memory=True)
        self.h_out = torch.empty((T, H), dtype=torch.float32, pin_memory=True)
        self.uses = np.zeros((L, E), dtype=np.int64)   # selections per (layer, expert) seen by this step
        self.host_sets = [[] for _ in range(L)]
        self.uploaded = [[] for _ in range(L)]
        self.host_ms = 0.0

    def calibrate(self, layer=0, n_rec=4):
        """Measure B_link (device-side fetch of records from pinned host memory)
        and B_host (host forward over records, one token); set q."""
        d, E, T = self.desc, self.desc.n_experts, self.T
        n_rec = min(n_rec, E, self.n_slots)
        ml = torch.tensor([n_rec] + [v for e in range(n_rec) for v in (e, e)], dtype=torch.int32, device="cuda")
        st = torch.cuda.current_stream()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ftmoe.ft_expert_fetch(self.pool, d.expert_stride, self.fetch_bytes, E, self.n_slots, self.src_dev[layer],
                              ml[1:], ml[:1], n_rec, stream=st)  # warm
        a.record(st)
        ftmoe.ft_expert_fetch(self.pool, d.expert_stride, self.fetch_bytes, E, self.n_slots, self.src_dev[layer],
                              ml[1:], ml[:1], n_rec, stream=st)
        b.record(st)
        torch.cuda.synchronize()
        b_link = n_rec * self.rec / (a.elapsed_time(b) * 1e-3)
        # the table no longer matches the pool's slots 0..n_rec-1: the caller
        # calibrates before the first lookup (the cold table has no residents)
        ids = np.array([[e % E for e in range(d.top_k)]], dtype=np.int32)
        gates = np.full((1, d.top_k), 1.0 / d.top_k, dtype=np.float32)
        x = np.zeros((1, d.hidden), dtype=np.uint16 if d.act_dtype == 1 else np.float32)
        out = np.empty((1, d.hidden), dtype=np.float32)
        ftmoe.ft_moe_forward_host(d, x, ids, gates, self.src_host[layer], out, n_threads=self.n_threads)
        t0 = time.perf_counter()
        ftmoe.ft_moe_forward_host(d, x, ids, gates, self.src_host[layer], out, n_threads=self.n_threads)
        b_host = d.top_k * self.rec / (time.perf_counter() - t0)
        self.q = b_host / (b_host + b_link)
        return {"link_gbs": b_link / 1e9, "host_gbs": b_host / 1e9, "q": self.q}

    def step(self, x, bias=None):
        """One step over every layer on the current stream (host-driven: one
        synchronisation per layer, after the residency probe)."""
        d, T, k, E = self.desc, self.T, self.desc.top_k, self.desc.n_experts
        st = torch.cuda.current_stream()
        q = 0.0 if self.q is None else self.q
        self.host_ms = 0.0
        for l in range(self.L):
            ml = self.mlist[l]
            ftmoe.ft_moe_route(d, x[l], self.routers[l], self.ids[l], self.gates[l],
                               sel_bias=None if bias is None else bias[l], workspace=self.rws, stream=st)
            ftmoe.ft_slot_probe(self.table, l, self.ids[l], self.res[l], stream=st)
            self.h_ids.copy_(self.ids[l], non_blocking=True)
            self.h_gates.copy_(self.gates[l], non_blocking=True)
            self.h_res.copy_(self.res[l], non_blocking=True)
            self.h_x.copy_(x[l].view(self.h_x.dtype), non_blocking=True)
            st.synchronize()
            ids_h = self.h_ids.numpy()
            sel = np.unique(ids_h[(ids_h >= 0) & (ids_h < E)])
            self.uses[l, sel] += 1
            miss = sorted(set(int(e) for e in ids_h[self.h_res.numpy() == 0]))
            n_c = int(round(q * len(miss)))
            # the host takes the misses selected least often so far (ties:
            # higher id): rarely used experts are computed in place and do not
            # displace the cache's frequently used ones
            by_use = sorted(miss, key=lambda e: (self.uses[l, e], -e))
            C = sorted(by_use[:n_c])
            self.host_sets[l] = C
            self.uploaded[l] = [e for e in miss if e not in C]
            lk = ids_h.copy()
            if C:
                lk[np.isin(lk, C)] = -1
            self.h_lk[l].numpy()[:] = lk
            self.h_mask[l].numpy()[:] = (~_bitset(C, E)).view(np.int32)
            self.ids_lk[l].copy_(self.h_lk[l], non_blocking=True)
            self.mask[l].copy_(self.h_mask[l], non_blocking=True)
            ftmoe.ft_slot_lookup(self.table, l, self.ids_lk[l], self.slots[l], self.flags[l], ml[1:], ml[:1],
                                 stream=st)
            ftmoe.ft_expert_fetch(self.pool, d.expert_stride, self.fetch_bytes, E, self.n_slots, self.src_dev[l],
                                  ml[1:], ml[:1], T * k, stream=st)
            ftmoe.ft_moe_forward(d, x[l], self.ids[l], self.gates[l], self.pool, self.out[l], self.ws,
                                 slot_ids=self.slots[l], expert_mask=self.mask[l], stream=st)
            if C:
                # the host leg, while the device works through the calls above
                t0 = time.perf_counter()
                ftmoe.ft_moe_forward_host(d, self.h_x, self.h_ids, self.h_gates, self.src_host[l], self.h_out,
                                          expert_mask=_bitset(C, E), n_threads=self.n_threads)
                self.host_ms += (time.perf_counter() - t0) * 1e3
                self.part.copy_(self.h_out, non_blocking=True)
                ftmoe.ft_moe_add_partial(self.out[l], self.part, stream=st)
