"""The benchmark's command-line contract: one JSON line with the agreed keys,
exactly the requested number of timed steps, one GPU only."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=600):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=timeout, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2", timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_nonpositive_steps_are_refused():
    r = _bench("--steps", "0", timeout=120)
    assert r.returncode == 2


@pytest.mark.gpu
def test_json_line_contract():
    r = _bench("--steps", "13", "--warmup", "3", "--rounds", "1", "--no-cpu-baseline", "--no-prefill",
               "--no-variants", "--no-model-step", "--no-floors", "--no-warm-column")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 13 and d["warmup"] == 3
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert "workload" in d["config"]
    roof = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
