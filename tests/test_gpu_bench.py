"""bench.py end to end on the small workload (flat 2^20 parameters, W=4): it
prints one JSON line with the metric, the throughput, the roofline object of
the dominant kernel and the CPU baseline, and the figures agree with each
other (params/s from ms/step, the roofline fraction from its own fields); the
secondary measurements (kernel median and minimum, other tensors written
between steps, the MALL-warm step) are present in both layouts."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

from tests.gpu_util import torch_cuda

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_contract():
    torch_cuda()
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "C1", "--no-per-config",
                          "--steps", "20", "--warmup", "2"], capture_output=True, text=True, timeout=240)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = [l for l in out.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, out.stdout
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 2 and d["unit"] == "params/s"
    assert d["config"]["workload"].startswith("flat 2^20") and d["config"]["shard_params"] == 262144
    assert abs(d["value"] - 262144 / (d["ms_per_step"] * 1e-3)) <= 1e-6 * d["value"]
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-12
    assert abs(r["achieved"] - r["algorithmic_bytes_per_launch"] / (r["kernel_ms"] * 1e-3) / 1e9) < 1e-6 * r["achieved"]
    assert 0 < r["frac"] < 1.0
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["single_thread"]["cores"] == 1
    assert set(d["layouts"]) == {"arena", "packed"} and "graph" in d
    for k in ("reduce", "update"):   # each kernel's mean, median and minimum of its K durations
        kk = d["kernels"][k]
        assert 0 < kk["ms_min"] <= kk["ms_median"] and kk["ms_min"] <= kk["ms"], (k, kk)
    for lay in ("arena", "packed"):
        e = d["layouts"][lay]
        o = e["other_tensors"]   # the step's kernels with 4 GiB of other writes before each step
        assert o["written_per_step_bytes"] == 4 << 30 and o["kernels_ms"] > 0, (lay, o)
        assert ("gaps" in o["where"]) == (lay == "arena"), o["where"]
        assert e["mall_warm_ms_per_step"] > 0   # the rotated workload's steps on one copy
