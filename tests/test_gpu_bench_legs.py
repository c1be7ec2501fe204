"""Every leg of bench.py runs on the GPU and prints one well-formed JSON line:
the verify step, prefill, the draft head, attention, and the decode-loop cost
model (a few steps each; the numbers themselves are not judged here)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.gpu


def _run(*args):
    print(f"[bench leg] {' '.join(args)}", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=400)
    assert r.returncode == 0, r.stderr[-3000:]
    return json.loads(r.stdout.strip().splitlines()[-1])


@pytest.mark.parametrize("wl", ["decode_b1", "prefill_8pages", "draft_b1", "attn_b1"])
def test_bench_leg(wl):
    line = _run("--workload", wl, "--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in line, key
    assert line["value"] > 0 and line["n_gpus"] == 1 and line["config"]["workload"] == wl
    roof = line["roofline"]
    assert roof["achieved"] > 0 and 0 < roof["frac"] < 1 and roof["bound"] in ("hbm", "mfma")
    if wl.startswith("attn"):
        assert 0 < line["attention"]["frac"] < 1


def test_bench_cost_model():
    line = _run("--workload", "decode_b1", "--cost-model", "--steps", "3", "--warmup", "1")
    rows = line["cost_model"]["rows"]
    assert [r["K"] for r in rows] == [0, 1, 2, 3]
    assert all(r["eager_us"] > 0 and r["graph_us"] > 0 for r in rows)
    assert all("loop_eager_us" in r for r in rows)
