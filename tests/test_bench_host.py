"""Host logic of bench.py (no GPU): the one-GPU contract, the defaults, the
fields every result line carries, and the measured-traffic lookups that
report null for any other workload or changed kernel source."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_defaults_finish_within_minutes(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert a.gpus == 1 and a.batch == 1 and a.workload == "decode_bf16_h2048_e128"
    assert a.steps <= 500 and a.warmup <= 100 and not a.single_batch and not a.eager


def test_result_line_fields():
    class A:
        steps, warmup = 7, 3
    r = bench._base_result(A(), 123.456, "tokens/s", 1.5, {"workload": "w"}, "bf16")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config"):
        assert key in r
    assert r["n_gpus"] == 1 and r["higher_is_better"] is True and r["vs_baseline"] is None
    assert r["data"] == "synthetic" and r["value"] == 123.5 and r["config"]["workload"] == "w"


@pytest.mark.parametrize("name,batch", [("decode_bf16_h2048_e128", 2), ("decode_nvfp4_h6144_e256", 1),
                                        ("tiny_f32", 1)])
def test_decode_traffic_only_for_the_measured_workload(name, batch):
    assert bench.measured_decode_traffic(name, batch) is None


def test_prefill_traffic_only_for_the_measured_workload():
    assert bench.measured_prefill_traffic("prefill_mxfp4_h4096_e256", 4096) is None
    assert bench.measured_prefill_traffic("decode_bf16_h2048_e128", 8192) is None


def test_traffic_tables_are_keyed_by_source_hashes():
    for key, v in bench.DECODE_TRAFFIC.items():
        assert len(key) == 16 and int(key, 16) >= 0 and v > 0
    for key, v in bench.PREFILL_TRAFFIC.items():
        assert key[0] in bench.PREFILL_WORKLOADS and key[1] in (1, 2)
        assert len(key) == 3 and len(key[2]) == 16 and int(key[2], 16) >= 0 and v > 0
    # the keys cover the headers the kernels include, not only their .hip files
    for srcs in [bench.DECODE_SRCS] + list(bench.PREFILL_SRCS.values()):
        names = [os.path.basename(p) for p in srcs]
        assert "common.hpp" in names and "internal.hpp" in names and "ft_moe.h" in names
        assert all(os.path.exists(p) for p in srcs)
    # a figure, when reported, is within a few per cent of the workload's design bytes
    d = bench.measured_decode_traffic("decode_bf16_h2048_e128", 1)
    if d is not None:
        assert 1.0 <= d / 75_509_760 <= 1.05
    for terms in (1, 2):
        p = bench.measured_prefill_traffic("prefill_mxfp4_h4096_e256", 8192, terms)
        if p is not None:  # at least the weights, activations and outputs; the intermediates on top
            assert 1.0 <= p / 3_620_000_000 <= 1.7
    p = bench.measured_prefill_traffic("prefill_bf16_h2048_e128", 8192)
    if p is not None:  # weights 1.208 GB, x 33.6 MB, out 67.1 MB, h and y written and read: 2.05 GB by design
        assert 1.0 <= p / 2_046_000_000 <= 1.5
    p = bench.measured_prefill_traffic("prefill_nvfp4_h6144_e256", 8192)
    if p is not None:  # weights 5.44 GB, x 100.7 MB, out 201.3 MB, h and y written and read: 7.89 GB by design
        assert 1.0 <= p / 7_890_000_000 <= 1.5
