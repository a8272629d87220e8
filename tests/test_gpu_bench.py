"""GPU: the benchmark's JSON line on a small workload.

``bench.py --config 1`` (3 ragged requests) with a few steps and a short
CPU baseline, in a child process: one JSON line with the metric, the step
time, the roofline of the attention kernel (its own events), the CPU oracle
baseline, the achievable peak of a plain streaming read (a 4 GiB buffer and
the step's own bytes, cold) and the context figures, each consistent with
the others.
"""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_of_a_small_workload():
    print("bench.py --config 1 --steps 5 --warmup 2 --cpu-budget 1 --no-graph", flush=True)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "1",
                          "--steps", "5", "--warmup", "2", "--cpu-budget", "1", "--no-graph"],
                         capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    d = json.loads(res.stdout.strip().splitlines()[-1])
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["vs_baseline"] is None
    assert d["config"]["workload"].startswith("tiny_ragged") and d["config"]["batch"] == 3
    assert d["dtype"] == "f32" and d["data"] == "synthetic"
    alg = d["algorithmic_bytes_per_step"]
    # value = algorithmic bytes over the step time
    assert d["value"] > 0
    assert abs(d["value"] - alg / (d["ms_per_step"] * 1e-3) / 1e9) <= 0.02 * d["value"] + 0.01
    attn = d["kernel_ms"]["attention"]
    assert 0 < attn <= d["ms_per_step"] * 1.05
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert abs(r["achieved"] - alg / (attn * 1e-3) / 1e9) <= 0.02 * r["achieved"] + 0.01
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    ap = d["achievable_peak"]
    assert ap["bytes"] == 4 << 30 and 1000 < ap["GB/s"] < 8000
    at = ap["at_step_bytes"]
    assert at["bytes"] == alg // 16 * 16 and at["regions"] >= 2 and at["us"] > 0
    assert abs(r["frac_of_plain_read_at_step_bytes"] - r["achieved"] / at["GB/s"]) < 1e-3
    assert d["context"]["attention_flop_per_byte_here"] > 0
