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
