"""bench.py's output contract on short runs of two workloads (GPU).

bench.py runs in a child process, as the driver runs it: one JSON line with
the metric, the per-step time, the roofline of the dominant kernel (and, on
prefill lines, the executed MFMA work beside it).
"""
import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
           "--no-cpu-baseline", *args]
    print(" ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def _common(d, metric, unit):
    assert d["metric"] == metric and d["unit"] == unit
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["data"].startswith("synthetic")
    rf = d["roofline"]
    assert rf["bound"] in ("mfma", "hbm") and 0 < rf["frac"] < 1
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3


def test_bench_prefill_line():
    d = _bench("--workload", "flat_prefill_1x1024_h4kv1_top4")
    _common(d, "selected-block attention TFLOP/s", "TFLOP/s")
    assert d["config"]["workload"] == "flat_prefill_1x1024_h4kv1_top4"
    ex = d["roofline"]["executed"]
    # every selected FLOP lies in a computed slot-block
    assert ex["flops"] >= d["work"]["attention_flops"] > 0
    assert 0 < ex["selected_share"] <= 1


def test_bench_decode_line():
    d = _bench("--workload", "paged_decode_e2m1_b128_h16kv1_top16")
    _common(d, "KV GB/s", "GB/s")
    assert d["config"]["workload"] == "paged_decode_e2m1_b128_h16kv1_top16"
    assert d["roofline"]["bound"] == "hbm" and d["roofline"]["peak"] == 8000.0
