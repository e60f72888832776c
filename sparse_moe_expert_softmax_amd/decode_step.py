"""One decode step through the global expert cache with miss handling on the
device, eager or as one captured HIP graph.

Per MoE layer, on one stream: route, slot lookup, fetch of the missed
records straight from pinned host memory (`ft_expert_fetch`), forward.  The
miss list and its count stay in device memory, so no call waits for the
host, nothing is allocated and nothing is read back: the whole step can be
captured once and replayed with each step's activations (and selection bias)
staged into fixed input buffers.  The pages keep cache control inside the
captured model forward (FreeToken explainer page, "how" section); here the
captured unit is the MoE side of a step.

This is argument plumbing around the C entry points; every step of the
layer runs in the library's kernels."""
import torch

from . import ftmoe
from .configs import BF16, F32


class DeviceFetchStep:
    """Fixed buffers and the launch sequence of one step over `n_layers`
    layers at `n_tokens` tokens.

    Inputs staged by the caller before each run: `x[l]` (activations of layer
    l, the descriptor's act dtype) and, if `with_bias`, `bias[l]` (fp32
    [T, E], selection only).  Outputs after each run: `ids`, `gates`,
    `slots`, `flags`, `mlist[l]` = [n_miss, (expert, slot) ...] and `out[l]`.
    `layer_src[l]` is a device int64 tensor of layer l's pinned host record
    addresses.  `table` was set up by ft_slot_table_init for `n_layers`
    layers and `n_slots` slots; `pool` is [>= n_slots, expert_stride] bytes.
    The slot table and pool belong to this object's stream while a step
    runs."""

    def __init__(self, desc, n_layers, n_tokens, table, n_slots, pool, record_bytes, routers, layer_src,
                 with_bias=True):
        H, E, k = desc.hidden, desc.n_experts, desc.top_k
        L, T = n_layers, n_tokens
        if len(routers) != L or len(layer_src) != L:
            raise ValueError("one router and one host address table per layer")
        if pool.dim() != 2 or pool.shape[0] < n_slots or pool.shape[1] * pool.element_size() < desc.expert_stride:
            raise ValueError(f"pool must hold {n_slots} records of {desc.expert_stride} bytes")
        if table.numel() * table.element_size() < ftmoe.ft_slot_table_bytes(L, E, n_slots):
            raise ValueError("slot table smaller than ft_slot_table_bytes(n_layers, n_experts, n_slots)")
        self.desc, self.L, self.T = desc, L, T
        self.table, self.pool, self.rec = table, pool, record_bytes
        self.n_slots = n_slots
        self.routers, self.layer_src = routers, layer_src
        act = {F32: torch.float32, BF16: torch.bfloat16}[desc.act_dtype]
        dev = pool.device
        self.x = torch.zeros((L, T, H), dtype=act, device=dev)
        self.bias = torch.zeros((L, T, E), dtype=torch.float32, device=dev) if with_bias else None
        self.ids = torch.empty((L, T, k), dtype=torch.int32, device=dev)
        self.gates = torch.empty((L, T, k), dtype=torch.float32, device=dev)
        self.slots = torch.empty((L, T, k), dtype=torch.int32, device=dev)
        self.flags = torch.empty((L, T, k), dtype=torch.uint8, device=dev)
        self.mlist = torch.empty((L, 2 * T * k + 1), dtype=torch.int32, device=dev)
        self.out = torch.empty((L, T, H), dtype=torch.float32, device=dev)
        self.ws = torch.empty(max(ftmoe.ft_moe_workspace_bytes(desc, T), 256), dtype=torch.uint8, device=dev)
        self.rws = torch.empty(max(ftmoe.ft_route_workspace_bytes(desc, T), 256), dtype=torch.uint8, device=dev)
        self.graph = None

    def enqueue(self, stream=None):
        """Launch the step's calls on `stream` (default: the current stream)."""
        s = torch.cuda.current_stream() if stream is None else stream
        d, T, k = self.desc, self.T, self.desc.top_k
        for l in range(self.L):
            ml = self.mlist[l]
            ftmoe.ft_moe_route(d, self.x[l], self.routers[l], self.ids[l], self.gates[l],
                               sel_bias=None if self.bias is None else self.bias[l], workspace=self.rws, stream=s)
            ftmoe.ft_slot_lookup(self.table, l, self.ids[l], self.slots[l], self.flags[l], ml[1:], ml[:1], stream=s)
            ftmoe.ft_expert_fetch(self.pool, d.expert_stride, self.rec, d.n_experts, self.n_slots, self.layer_src[l],
                                  ml[1:], ml[:1], T * k, stream=s)
            ftmoe.ft_moe_forward(d, self.x[l], self.ids[l], self.gates[l], self.pool, self.out[l], self.ws,
                                 slot_ids=self.slots[l], stream=s)

    def capture(self):
        """Capture the step once; later `run()` calls replay it.  Capturing
        launches nothing, so the table and pool are untouched."""
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
        """One step on the current stream: the captured graph if there is one."""
        if self.graph is not None:
            self.graph.replay()
        else:
            self.enqueue()
