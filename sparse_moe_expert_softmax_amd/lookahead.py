"""One decode step through the global expert cache with look-ahead prefetch:
while layer l computes, the experts layer l+1 is predicted to use are
already being copied into the cache.

The pages predict the experts the next layer will need and page them in
ahead of use (FreeToken blog page, predictive expert paging).  The
prediction here is the plainest one: layer l+1's own router applied to layer
l's input, whose top-k is the predicted set.  It is good to the extent that
the router input changes little from one layer to the next (a residual
stream); the synthetic inputs for it come from
`synth.layer_correlated_activations`.

Per layer l, on the step's stream: route (x_l), slot lookup, on-device fetch
of the misses (`ft_expert_fetch`); then, if there is a next layer, the
prediction: layer l+1's router on x_l, a lookup of the predicted ids for
layer l+1 (which stamps them and places the missing ones), and, on a side
stream, the fetch of those predicted misses, which overlaps with layer l's
forward and layer l+1's router; the step's stream waits for that fetch
before layer l+1's lookup, so no slot being filled is ever handed out or
evicted.  Layer l+1's real lookup then finds the correctly predicted experts
resident.  Nothing is read back or allocated, so the step can be captured as
one HIP graph (two streams joined by events).

The prediction's own lookup is part of the cache's history, so the LRU state
is that of the sequence (predicted ids of l+1, real ids of l+1) per layer.

Argument plumbing around the C entry points only."""
import torch

from . import ftmoe


class LookaheadStep:
    """Fixed buffers and the launch sequence of one step over `n_layers`
    layers at `n_tokens` tokens, with (lookahead=True) or without the
    prediction.  Inputs staged before each run: x [L, T, H].  Outputs after
    each run: ids, gates, slots, out [L, ...], pred_ids [L, T, k] (row l =
    the prediction for layer l, made at layer l-1; row 0 unused), and
    mlist[l] / pmlist[l] = [n_miss, (expert, slot) ...] of the real and the
    predicted lookups."""

    def __init__(self, desc, n_layers, n_tokens, table, n_slots, pool, record_bytes, routers, layer_src,
                 lookahead=True):
        H, E, k = desc.hidden, desc.n_experts, desc.top_k
        L, T = n_layers, n_tokens
        if len(routers) != L or len(layer_src) != L:
            raise ValueError("one router and one host address table per layer")
        if pool.dim() != 2 or pool.shape[0] < n_slots or pool.shape[1] * pool.element_size() < desc.expert_stride:
            raise ValueError(f"pool must hold {n_slots} records of {desc.expert_stride} bytes")
        self.desc, self.L, self.T, self.lookahead = desc, L, T, lookahead
        self.table, self.pool, self.n_slots = table, pool, n_slots
        self.fetch_bytes = (record_bytes + 15) // 16 * 16  # the device copy moves 16-byte pieces
        if self.fetch_bytes > desc.expert_stride:
            raise ValueError("record bytes rounded to 16 exceed the expert stride")
        self.routers, self.layer_src = routers, layer_src
        dev = pool.device
        act = torch.bfloat16 if desc.act_dtype == 1 else torch.float32
        self.x = torch.zeros((L, T, H), dtype=act, device=dev)
        self.ids = torch.empty((L, T, k), dtype=torch.int32, device=dev)
        self.gates = torch.empty((L, T, k), dtype=torch.float32, device=dev)
        self.slots = torch.empty((L, T, k), dtype=torch.int32, device=dev)
        self.flags = torch.empty((L, T, k), dtype=torch.uint8, device=dev)
        self.mlist = torch.empty((L, 2 * T * k + 1), dtype=torch.int32, device=dev)
        self.pred_ids = torch.full((L, T, k), -1, dtype=torch.int32, device=dev)
        self.pred_gates = torch.empty((L, T, k), dtype=torch.float32, device=dev)
        self.pslots = torch.empty((L, T, k), dtype=torch.int32, device=dev)
        self.pflags = torch.empty((L, T, k), dtype=torch.uint8, device=dev)
        self.pmlist = torch.zeros((L, 2 * T * k + 1), dtype=torch.int32, device=dev)
        self.out = torch.empty((L, T, H), dtype=torch.float32, device=dev)
        self.ws = torch.empty(max(ftmoe.ft_moe_workspace_bytes(desc, T), 256), dtype=torch.uint8, device=dev)
        self.rws = torch.empty(max(ftmoe.ft_route_workspace_bytes(desc, T), 256), dtype=torch.uint8, device=dev)
        self.side = torch.cuda.Stream(device=dev)
        self.graph = None

    def enqueue(self, stream=None):
        s = torch.cuda.current_stream() if stream is None else stream
        d, T, k, E = self.desc, self.T, self.desc.top_k, self.desc.n_experts
        prefetched = None
        for l in range(self.L):
            ml = self.mlist[l]
            ftmoe.ft_moe_route(d, self.x[l], self.routers[l], self.ids[l], self.gates[l], workspace=self.rws, stream=s)
            if prefetched is not None:
                s.wait_event(prefetched)  # the predicted records have landed
            ftmoe.ft_slot_lookup(self.table, l, self.ids[l], self.slots[l], self.flags[l], ml[1:], ml[:1], stream=s)
            ftmoe.ft_expert_fetch(self.pool, d.expert_stride, self.fetch_bytes, E, self.n_slots, self.layer_src[l],
                                  ml[1:], ml[:1], T * k, stream=s)
            prefetched = None
            if self.lookahead and l + 1 < self.L:
                p, pml = l + 1, self.pmlist[l + 1]
                ftmoe.ft_moe_route(d, self.x[l], self.routers[p], self.pred_ids[p], self.pred_gates[p],
                                   workspace=self.rws, stream=s)
                ftmoe.ft_slot_lookup(self.table, p, self.pred_ids[p], self.pslots[p], self.pflags[p], pml[1:],
                                     pml[:1], stream=s)
                ev = torch.cuda.Event()
                ev.record(s)
                self.side.wait_event(ev)
                ftmoe.ft_expert_fetch(self.pool, d.expert_stride, self.fetch_bytes, E, self.n_slots,
                                      self.layer_src[p], pml[1:], pml[:1], T * k, stream=self.side)
                prefetched = torch.cuda.Event()
                prefetched.record(self.side)
            ftmoe.ft_moe_forward(d, self.x[l], self.ids[l], self.gates[l], self.pool, self.out[l], self.ws,
                                 slot_ids=self.slots[l], stream=s)

    def capture(self):
        g = torch.cuda.CUDAGraph()
        cur = torch.cuda.current_stream()
        cap = torch.cuda.Stream()
        cap.wait_stream(cur)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                self.enqueue(torch.cuda.current_stream())
        cur.wait_stream(cap)
        self.graph = g

    def run(self):
        if self.graph is not None:
            self.graph.replay()
        else:
            self.enqueue()
