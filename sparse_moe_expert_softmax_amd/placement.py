"""Expert placement policies at equal cache capacity, compared on a routing
trace: the library's global LRU over all layers, a per-layer split with LRU
inside each layer, and a static set profiled on the first steps of the trace.

The pages compare their global LRU against a static split between devices
and a prefill-based placement on the same routing trace and cache capacity
(FreeToken architecture guide, evaluation passage; explainer, "how").  The
two LRU policies run the library's slot-table kernel (ft_slot_lookup), one
table for all layers or one per layer; the static policy is a count over the
profiled steps.  Every function returns misses per (step, layer): distinct
selected experts not resident when the layer looks them up."""
import numpy as np

from . import ftmoe


def lru_misses(torch, trace: np.ndarray, n_experts: int, n_slots: int, per_layer: bool) -> np.ndarray:
    """trace [steps, layers, n] expert ids -> misses [steps, layers] (int32) of
    the global LRU table (n_slots slots shared by all layers) or, with
    per_layer, of one table of n_slots // layers slots per layer.  A negative
    entry marks an exhausted pool."""
    n_steps, L, n = trace.shape
    ids_all = torch.from_numpy(np.ascontiguousarray(trace).astype(np.int32)).cuda()
    slots = torch.empty(n, dtype=torch.int32, device="cuda")
    flags = torch.empty(n, dtype=torch.uint8, device="cuda")
    mlist = torch.empty(2 * n, dtype=torch.int32, device="cuda")
    if per_layer:
        s_l = n_slots // L
        tabs = [torch.zeros(ftmoe.ft_slot_table_bytes(1, n_experts, s_l), dtype=torch.uint8, device="cuda")
                for _ in range(L)]
        for t_ in tabs:
            ftmoe.ft_slot_table_init(t_, 1, n_experts, s_l)
    else:
        tabs = [torch.zeros(ftmoe.ft_slot_table_bytes(L, n_experts, n_slots), dtype=torch.uint8, device="cuda")]
        ftmoe.ft_slot_table_init(tabs[0], L, n_experts, n_slots)
    nm = torch.zeros((n_steps, L), dtype=torch.int32, device="cuda")
    for s in range(n_steps):
        for l in range(L):
            tab, lay = (tabs[l], 0) if per_layer else (tabs[0], l)
            ftmoe.ft_slot_lookup(tab, lay, ids_all[s, l], slots, flags, mlist, nm[s, l:l + 1])
    return nm.cpu().numpy()


def profiled_static_misses(trace: np.ndarray, n_experts: int, n_slots: int, profile_steps: int) -> np.ndarray:
    """The n_slots (layer, expert) keys selected in the most profiled steps
    (ties: lower layer * E + expert first) stay resident; every other selected
    key misses each time.  -> misses [steps, layers]."""
    n_steps, L, _ = trace.shape
    cnt = np.zeros((L, n_experts), dtype=np.int64)
    for s in range(profile_steps):
        for l in range(L):
            cnt[l, np.unique(trace[s, l])] += 1
    resident = np.zeros(L * n_experts, dtype=bool)
    resident[np.argsort(-cnt.ravel(), kind="stable")[:n_slots]] = True
    out = np.zeros((n_steps, L), dtype=np.int64)
    for s in range(n_steps):
        for l in range(L):
            u = np.unique(trace[s, l])
            out[s, l] = int((~resident[l * n_experts + u]).sum())
    return out


def distinct_selected(trace: np.ndarray) -> np.ndarray:
    """Distinct experts per (step, layer)."""
    n_steps, L, _ = trace.shape
    return np.array([[len(np.unique(trace[s, l])) for l in range(L)] for s in range(n_steps)])
