"""Thin ctypes binding of ``libftmoe.so`` (declared in ``include/ft_moe.h``).

Argument marshalling only: the functions take torch tensors (device memory,
pinned host memory) and torch streams, pass raw pointers to the C ABI and
raise on a non-OK status.  Every step of the layer runs in the HIP library;
there is no fallback.  The names follow the C entry points.
"""
import ctypes
import os

import torch

from .configs import MoEConfig

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libftmoe.so")

FT_OK, FT_EINVAL, FT_EUNSUPPORTED, FT_EPOOL, FT_EHIP, FT_EWORKSPACE = 0, -1, -2, -3, -4, -5
STATUS_NAMES = {0: "FT_OK", -1: "FT_EINVAL", -2: "FT_EUNSUPPORTED", -3: "FT_EPOOL", -4: "FT_EHIP",
                -5: "FT_EWORKSPACE"}


class FtError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("act_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
                ("router_dtype", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("expert_stride", ctypes.c_int64), ("act_terms", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class PrefillPipelineState(ctypes.Structure):
    """ft_prefill_pipeline (caller-owned state of the double-buffered prefill)."""
    _fields_ = [("layer_buf", ctypes.c_void_p * 2), ("expert_stride", ctypes.c_int64),
                ("record_bytes", ctypes.c_int64), ("n_experts", ctypes.c_int32), ("n_done", ctypes.c_int32),
                ("n_uploaded", ctypes.c_int32), ("reserved", ctypes.c_int32), ("compute_stream", ctypes.c_void_p),
                ("copy_stream", ctypes.c_void_p), ("ready", ctypes.c_void_p * 2), ("freed", ctypes.c_void_p * 2)]


_lib = None
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "ft_record_bytes": (_sz, [_i32, _i32, _i32]),
    "ft_route_workspace_bytes": (_sz, [ctypes.POINTER(Desc), _i32]),
    "ft_moe_route": (ctypes.c_int, [ctypes.POINTER(Desc), _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ft_slot_table_bytes": (_sz, [_i32, _i32, _i32]),
    "ft_slot_table_init": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp]),
    "ft_slot_lookup": (ctypes.c_int, [_vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _vp]),
    "ft_expert_upload": (ctypes.c_int, [_vp, _i64, _i64, ctypes.POINTER(_i32), ctypes.POINTER(_vp), _i32, _vp, _vp]),
    "ft_expert_fetch": (ctypes.c_int, [_vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _i32, _vp]),
    "ft_moe_workspace_bytes": (_sz, [ctypes.POINTER(Desc), _i32]),
    "ft_moe_forward": (ctypes.c_int, [ctypes.POINTER(Desc), _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ft_moe_route_forward_workspace_bytes": (_sz, [ctypes.POINTER(Desc), _i32]),
    "ft_moe_route_forward": (ctypes.c_int, [ctypes.POINTER(Desc), _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                            _sz, _vp]),
    "ft_moe_route_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(Desc), _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                                    _vp, _vp]),
    "ft_prefill_pipeline_start": (ctypes.c_int, [ctypes.POINTER(PrefillPipelineState), ctypes.POINTER(_vp)]),
    "ft_prefill_pipeline_layer": (ctypes.c_int, [ctypes.POINTER(PrefillPipelineState), ctypes.POINTER(_vp),
                                                 ctypes.POINTER(Desc), _vp, _i32, _vp, _vp, _vp, _vp, _vp, _sz]),
    "ft_slot_probe": (ctypes.c_int, [_vp, _i32, _vp, _i32, _vp, _vp]),
    "ft_moe_forward_host": (ctypes.c_int, [ctypes.POINTER(Desc), _vp, _i32, _vp, _vp, ctypes.POINTER(_vp), _vp, _vp,
                                           _i32]),
    "ft_moe_add_partial": (ctypes.c_int, [_vp, _vp, _i64, _vp]),
    "ft_last_error": (ctypes.c_char_p, []),
}
EXPORTED = tuple(_SIGS)


def lib():
    """Load the built library; raise if it is missing (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_moe_expert_softmax_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int):
    if rc != FT_OK:
        raise FtError(rc, lib().ft_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_desc(cfg: MoEConfig, expert_stride: int = None, act_terms: int = 0) -> Desc:
    from .synth import record_stride
    stride = record_stride(cfg.hidden, cfg.inter, cfg.w_dtype) if expert_stride is None else expert_stride
    return Desc(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.act_dtype, cfg.w_dtype, cfg.router_dtype,
                1 if cfg.renormalize else 0, stride, act_terms, 0)


def ft_record_bytes(hidden: int, inter: int, w_dtype: int) -> int:
    return int(lib().ft_record_bytes(hidden, inter, w_dtype))


def ft_route_workspace_bytes(desc: Desc, n_tokens: int) -> int:
    return int(lib().ft_route_workspace_bytes(ctypes.byref(desc), n_tokens))


def ft_moe_route(desc: Desc, x, w_router, topk_ids, topk_gates, sel_bias=None, logits=None, workspace=None,
                 stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ft_moe_route(ctypes.byref(desc), _ptr(x), x.shape[0], _ptr(w_router), _ptr(sel_bias),
                              _ptr(topk_ids), _ptr(topk_gates), _ptr(logits), _ptr(workspace), ws_bytes,
                              _stream(stream)))


def ft_slot_table_bytes(n_layers: int, n_experts: int, n_slots: int) -> int:
    return int(lib().ft_slot_table_bytes(n_layers, n_experts, n_slots))


def ft_slot_table_init(table, n_layers: int, n_experts: int, n_slots: int, stream=None):
    _check(lib().ft_slot_table_init(_ptr(table), n_layers, n_experts, n_slots, _stream(stream)))


def ft_slot_lookup(table, layer: int, topk_ids, slot_ids, miss_flags, miss_list, n_miss, stream=None):
    _check(lib().ft_slot_lookup(_ptr(table), layer, _ptr(topk_ids), topk_ids.numel(), _ptr(slot_ids),
                                _ptr(miss_flags), _ptr(miss_list), _ptr(n_miss), _stream(stream)))


def ft_expert_upload(pool, expert_stride: int, record_bytes: int, slots, host_ptrs, stream=None, done_event=None):
    """slots: list of ints; host_ptrs: list of integer host addresses (pinned)."""
    n = len(slots)
    arr_s = (_i32 * max(n, 1))(*slots)
    arr_p = (_vp * max(n, 1))(*host_ptrs)
    ev = None
    if done_event is not None:
        if not done_event.cuda_event:  # torch creates the HIP event lazily: create it on this stream first
            done_event.record(torch.cuda.current_stream() if stream is None else stream)
        ev = ctypes.c_void_p(done_event.cuda_event)
    _check(lib().ft_expert_upload(_ptr(pool), expert_stride, record_bytes, arr_s, arr_p, n, _stream(stream), ev))


def ft_expert_fetch(pool, expert_stride: int, record_bytes: int, n_experts: int, n_slots: int, layer_src, miss_list,
                    n_miss, max_miss: int, stream=None):
    """layer_src: device int64 tensor [n_experts] of pinned host record addresses;
    miss_list / n_miss: the device tensors ft_slot_lookup wrote."""
    _check(lib().ft_expert_fetch(_ptr(pool), expert_stride, record_bytes, n_experts, n_slots, _ptr(layer_src),
                                 _ptr(miss_list), _ptr(n_miss), max_miss, _stream(stream)))


def ft_moe_workspace_bytes(desc: Desc, n_tokens: int) -> int:
    return int(lib().ft_moe_workspace_bytes(ctypes.byref(desc), n_tokens))


def ft_moe_forward(desc: Desc, x, topk_ids, topk_gates, pool, out, workspace, slot_ids=None, expert_mask=None,
                   stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().ft_moe_forward(ctypes.byref(desc), _ptr(x), x.shape[0], _ptr(topk_ids), _ptr(topk_gates),
                                _ptr(slot_ids), _ptr(pool), _ptr(expert_mask), _ptr(out), _ptr(workspace),
                                ws_bytes, _stream(stream)))


def ft_moe_route_forward_workspace_bytes(desc: Desc, n_tokens: int) -> int:
    return int(lib().ft_moe_route_forward_workspace_bytes(ctypes.byref(desc), n_tokens))


def ft_moe_route_forward(desc: Desc, x, w_router, topk_ids, topk_gates, pool, out, workspace, sel_bias=None,
                         expert_mask=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().ft_moe_route_forward(ctypes.byref(desc), _ptr(x), x.shape[0], _ptr(w_router), _ptr(sel_bias),
                                      _ptr(topk_ids), _ptr(topk_gates), _ptr(pool), _ptr(expert_mask), _ptr(out),
                                      _ptr(workspace), ws_bytes, _stream(stream)))


def ft_moe_route_forward_noalloc(desc: Desc, x, w_router, topk_ids, topk_gates, pool, out, sel_bias=None,
                                 expert_mask=None, stream=None):
    _check(lib().ft_moe_route_forward_noalloc(ctypes.byref(desc), _ptr(x), x.shape[0], _ptr(w_router),
                                              _ptr(sel_bias), _ptr(topk_ids), _ptr(topk_gates), _ptr(pool),
                                              _ptr(expert_mask), _ptr(out), _stream(stream)))


FT_NOALLOC_SCRATCH_BYTES = 32 << 20


def ft_prefill_pipeline_start(state: PrefillPipelineState, first_layer_ptrs):
    """first_layer_ptrs: list of n_experts integer addresses of pinned host records."""
    arr = (_vp * len(first_layer_ptrs))(*first_layer_ptrs)
    _check(lib().ft_prefill_pipeline_start(ctypes.byref(state), arr))


def ft_prefill_pipeline_layer(state: PrefillPipelineState, next_layer_ptrs, desc: Desc, x, w_router, topk_ids,
                              topk_gates, out, workspace):
    """next_layer_ptrs: list of pinned host record addresses, or None at the last layer."""
    arr = None if next_layer_ptrs is None else (_vp * len(next_layer_ptrs))(*next_layer_ptrs)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().ft_prefill_pipeline_layer(ctypes.byref(state), arr, ctypes.byref(desc), _ptr(x), x.shape[0],
                                           _ptr(w_router), _ptr(topk_ids), _ptr(topk_gates), _ptr(out),
                                           _ptr(workspace), ws_bytes))


def ft_slot_probe(table, layer: int, ids, resident, stream=None):
    _check(lib().ft_slot_probe(_ptr(table), layer, _ptr(ids), ids.numel(), _ptr(resident), _stream(stream)))


def _host_ptr(a):
    """Address of a host array: a CPU torch tensor or a numpy array."""
    if a is None:
        return None
    if hasattr(a, "data_ptr"):
        return ctypes.c_void_p(a.data_ptr())
    return ctypes.c_void_p(a.ctypes.data)


def ft_moe_forward_host(desc: Desc, x, topk_ids, topk_gates, record_ptrs, out, expert_mask=None, n_threads=0):
    """Host pointers throughout: x, topk_ids, topk_gates, out and expert_mask are
    CPU tensors or numpy arrays; record_ptrs is a list of n_experts integer
    host addresses (0 / None for experts that are not read)."""
    arr = (_vp * len(record_ptrs))(*[p or None for p in record_ptrs])
    _check(lib().ft_moe_forward_host(ctypes.byref(desc), _host_ptr(x), x.shape[0], _host_ptr(topk_ids),
                                     _host_ptr(topk_gates), arr, _host_ptr(expert_mask), _host_ptr(out), n_threads))


def ft_moe_add_partial(out, part, stream=None):
    _check(lib().ft_moe_add_partial(_ptr(out), _ptr(part), out.numel(), _stream(stream)))


def ft_last_error() -> str:
    return lib().ft_last_error().decode()
