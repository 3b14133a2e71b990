"""bench.py on the GPU: the graph-replay mode captures whole steps and reports
itself, on the float32 workload (the one whose eager step the host's launch
cost sets)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "smollm2_qkv_f32", "--steps",
                        "50", "--warmup", "5", "--warmup-seconds", "0.1", "--blocks", "1", "--no-cpu-baseline", *args],
                       capture_output=True, text=True, timeout=100)
    assert r.returncode == 0, r.stderr[-2000:]
    return json.loads(r.stdout.strip().splitlines()[-1])


@pytest.mark.gpu
def test_bench_graph_mode_reports_replayed_steps():
    d = _bench("--graph")
    assert d["launch"] == "hip graph replay"
    assert d["steps"] == 50 and d["ms_per_step"] > 0 and d["value"] > 0
    r = d["roofline"]
    assert r["launches_per_step"] == 1 and r["kernel_ms"] == d["ms_per_step"]
    # the unfused baseline and the hot blocks go through the same graph path
    assert d["unfused"]["ms_per_step"] > 0 and r["hot_ms_per_step"] > 0
    assert d["speedup_vs_unfused"] > 0


@pytest.mark.gpu
def test_bench_eager_mode_is_the_default():
    d = _bench()
    assert d["launch"] == "eager"
    assert d["ms_per_step"] > 0 and d["value"] > 0
