"""bench.py end to end on the GPU (a short run in a child process): exactly one JSON line on
stdout, with the fields and meanings of the benchmark line (one GPU, weak scaling, synthetic
data, the roofline of the prefill call with its fraction and counter traffic, the CPU
baseline of the oracle)."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    print("[gpu-case] bench.py --steps 2 --warmup 1 --no-extra --decode-steps 50", file=sys.stderr, flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
                        "--no-extra", "--cpu-sample-tokens", "2048", "--decode-steps", "50",
                        "--cpu-decode-steps", "2"],
                       capture_output=True, text=True, timeout=280, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["unit"] == "tokens/s" and d["value"] > 0 and d["ms_per_step"] > 0
    assert d["higher_is_better"] is True and d["scaling"] == "weak" and d["data"] == "synthetic"
    assert d["vs_baseline"] is None
    assert isinstance(d["config"], dict) and "workload" in d["config"]
    rl = d["roofline"]
    assert rl["bound"] == "hbm" and rl["unit"] == "GB/s" and rl["peak"] == 8000.0
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    # counter traffic is reported while the committed counters belong to this kernel source
    # (null otherwise); the split's records make it larger than the algorithmic bytes
    assert rl["traffic"] is None or rl["traffic"] > rl["algorithmic_bytes_per_launch"]
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["unit"] == "tokens/s"
    assert "2048 tokens" in cb["sample"]
    assert cb["decode"]["unit"] == "steps/s" and cb["decode"]["value"] > 0 and "2 consecutive steps" in cb["decode"]["sample"]
    # the decode block: consecutive steps between one pair of events, against 8 TB/s
    dec = d["decode"]
    assert "50 consecutive steps" in dec["protocol"] and d["config"]["decode"]["steps_per_step"] == 50
    assert abs(dec["frac"] - dec["achieved_gbs"] / dec["peak_gbs"]) < 1e-3
    assert abs(dec["steps_per_s"] * dec["avg_launch_us"] - 1e6) < 1e3
    # one step: one prefill call and 50 decode steps, all inside the step's time
    assert d["ms_per_step"] >= rl["avg_launch_ms"] + 50 * dec["avg_launch_us"] * 1e-3 * 0.99
