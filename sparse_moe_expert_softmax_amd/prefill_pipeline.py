"""The double-buffered prefill pipeline's device buffers, streams and events,
around the C entry points ft_prefill_pipeline_start / _layer.

While layer n computes from one device layer buffer, layer n+1's whole
expert set is copied from pinned host memory into the other on a side
stream (FreeToken explainer page, "how" section; architecture guide,
prefill passage).  This module only allocates the two buffers, the side
stream and the four events with torch and passes their addresses; the
sequencing (which buffer, which waits, which records) is the library's."""
import torch

from . import ftmoe


class PrefillPipeline:
    """Two [n_experts, expert_stride] device layer buffers on `compute_stream`
    (default: the current stream) with a side copy stream.

    start(first) enqueues layer 0's copy; layer(next, x, router, ...) runs
    one layer from the buffer its copy filled and starts the copy of `next`
    (None at the last layer).  Host records are lists of pinned host
    addresses, one per expert."""

    def __init__(self, desc, record_bytes, compute_stream=None):
        E, stride = desc.n_experts, desc.expert_stride
        self.desc = desc
        self.compute = torch.cuda.current_stream() if compute_stream is None else compute_stream
        self.copy = torch.cuda.Stream()
        self.bufs = [torch.empty((E, stride), dtype=torch.uint8, device="cuda") for _ in range(2)]
        self.ready = [torch.cuda.Event() for _ in range(2)]
        self.freed = [torch.cuda.Event() for _ in range(2)]
        for ev in self.ready:      # torch creates the HIP event at its first record
            ev.record(self.copy)
        for ev in self.freed:
            ev.record(self.compute)
        s = ftmoe.PrefillPipelineState()
        s.layer_buf[0], s.layer_buf[1] = self.bufs[0].data_ptr(), self.bufs[1].data_ptr()
        s.expert_stride, s.record_bytes, s.n_experts = stride, record_bytes, E
        s.compute_stream, s.copy_stream = self.compute.cuda_stream, self.copy.cuda_stream
        s.ready[0], s.ready[1] = self.ready[0].cuda_event, self.ready[1].cuda_event
        s.freed[0], s.freed[1] = self.freed[0].cuda_event, self.freed[1].cuda_event
        self.state = s

    def start(self, first_layer_ptrs):
        ftmoe.ft_prefill_pipeline_start(self.state, first_layer_ptrs)

    def layer(self, next_layer_ptrs, x, w_router, topk_ids, topk_gates, out, workspace):
        ftmoe.ft_prefill_pipeline_layer(self.state, next_layer_ptrs, self.desc, x, w_router, topk_ids, topk_gates,
                                        out, workspace)

    @property
    def n_done(self) -> int:
        return self.state.n_done
