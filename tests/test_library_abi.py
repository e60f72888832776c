"""CPU checks of the boundary: the library builds, loads, and exports every
entry point the C header declares (no compute calls without a GPU)."""
import ctypes
import os
import re

import pytest

from sparse_moe_expert_softmax_amd import ftmoe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    txt = open(os.path.join(ROOT, "include", "ft_moe.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(ft_[a-z_0-9]+)\s*\(", txt)))


def test_header_declares_the_entry_points():
    names = header_functions()
    for n in ("ft_moe_route", "ft_slot_lookup", "ft_moe_forward", "ft_expert_upload"):
        assert n in names


def test_library_exports_every_declared_symbol():
    if not os.path.exists(ftmoe.LIB_PATH):
        pytest.skip("library not built")
    L = ctypes.CDLL(ftmoe.LIB_PATH)
    for n in header_functions():
        assert hasattr(L, n), n
    assert set(header_functions()) == set(ftmoe.EXPORTED)


def test_size_queries_and_validation_without_gpu():
    if not os.path.exists(ftmoe.LIB_PATH):
        pytest.skip("library not built")
    from sparse_moe_expert_softmax_amd import synth
    from sparse_moe_expert_softmax_amd.configs import CONFIGS
    for cfg in CONFIGS.values():
        assert ftmoe.ft_record_bytes(cfg.hidden, cfg.inter, cfg.w_dtype) == synth.record_bytes(
            cfg.hidden, cfg.inter, cfg.w_dtype)
    d = ftmoe.make_desc(CONFIGS["tiny_f32"])
    assert ftmoe.ft_moe_workspace_bytes(d, 16) > 0
    assert ftmoe.ft_slot_table_bytes(43, 256, 2752) == 64 + 4 * (43 * 256 + 2752) + 4 * 2752
    bad = ftmoe.make_desc(CONFIGS["tiny_f32"])
    bad.top_k = 99
    assert ftmoe.ft_moe_workspace_bytes(bad, 16) == 0
    rc = ftmoe.lib().ft_moe_forward(ctypes.byref(bad), None, 4, None, None, None, None, None, None, None, 0, None)
    assert rc == ftmoe.FT_EINVAL and "top_k" in ftmoe.ft_last_error()
    rc = ftmoe.lib().ft_slot_lookup(None, 0, None, 4, None, None, None, None, None)
    assert rc == ftmoe.FT_EINVAL


def test_prefill_pipeline_refuses_bad_state_without_gpu():
    """Checks that run before any HIP call: missing buffers, equal streams,
    a layer whose copy was never enqueued."""
    if not os.path.exists(ftmoe.LIB_PATH):
        pytest.skip("library not built")
    assert ctypes.sizeof(ftmoe.PrefillPipelineState) == 96
    s = ftmoe.PrefillPipelineState()
    rc = ftmoe.lib().ft_prefill_pipeline_start(ctypes.byref(s), None)
    assert rc == ftmoe.FT_EINVAL and "layer buffers" in ftmoe.ft_last_error()
    s.layer_buf[0], s.layer_buf[1] = 4096, 8192
    s.ready[0] = s.ready[1] = s.freed[0] = s.freed[1] = 1
    s.expert_stride, s.record_bytes, s.n_experts = 4096, 4096, 2
    s.compute_stream = s.copy_stream = 7
    rc = ftmoe.lib().ft_prefill_pipeline_start(ctypes.byref(s), None)
    assert rc == ftmoe.FT_EINVAL and "copy_stream" in ftmoe.ft_last_error()
    s.copy_stream = 9
    from sparse_moe_expert_softmax_amd.configs import MXFP4, MoEConfig, BF16
    cfg = MoEConfig("abi_pipe", 99, hidden=256, inter=256, n_experts=2, top_k=1, act_dtype=BF16,
                    router_dtype=BF16, w_dtype=MXFP4, n_layers=1)
    d = ftmoe.make_desc(cfg, 4096)
    s.n_done, s.n_uploaded = 1, 1      # layer 1 was never uploaded
    buf = ctypes.create_string_buffer(64)
    rc = ftmoe.lib().ft_prefill_pipeline_layer(ctypes.byref(s), None, ctypes.byref(d), buf, 4, buf, buf, buf, buf,
                                               buf, 1 << 30)
    assert rc == ftmoe.FT_EINVAL and "not uploaded" in ftmoe.ft_last_error()


def test_probe_library_exports_and_refuses_bad_arguments_without_gpu():
    """The ceiling-probe library (benchmark only, not the MoE path) loads,
    exports its four launchers, and refuses bad arguments before any launch."""
    path = os.path.join(ROOT, "sparse_moe_expert_softmax_amd", "libftprobe.so")
    if not os.path.exists(path):
        pytest.skip("probe library not built")
    L = ctypes.CDLL(path)
    for n in ("ftp_stream_read", "ftp_empty", "ftp_mfma", "ftp_lds_dma"):
        assert hasattr(L, n), n
    buf = ctypes.create_string_buffer(64)
    p = ctypes.cast(buf, ctypes.c_void_p)
    assert L.ftp_stream_read(p, ctypes.c_int64(8), ctypes.c_int32(1), p, ctypes.c_int32(1), ctypes.c_int32(0), None) == -1
    assert L.ftp_stream_read(p, ctypes.c_int64(16), ctypes.c_int32(1), p, ctypes.c_int32(1), ctypes.c_int32(4), None) == -1
    assert L.ftp_empty(ctypes.c_int32(-1), None) == -1
    assert L.ftp_mfma(ctypes.c_int32(6), p, ctypes.c_int32(1), ctypes.c_int32(1), None) == -1
    assert L.ftp_lds_dma(p, ctypes.c_int64(100), p, ctypes.c_int32(1), ctypes.c_int32(1), None) == -1
