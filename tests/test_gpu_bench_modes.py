"""bench.py's modes run end to end and print one JSON line in the bench contract.

Each mode runs in a child process with two timed steps (no settling, no host
baseline), so this checks that the mode issues its calls and reports, not its speed.
"""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
        "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline"}


@pytest.mark.gpu
@pytest.mark.parametrize("mode", [
    [], ["--streams"], ["--cached-pooling"], ["--managed-window"], ["--ragged"],
    ["--rope-cap", "8"], ["--backward"], ["--serial"], ["--side-stream"], ["--no-ahead"],
])
def test_bench_mode_prints_contract_line(mode):
    print("bench mode", mode, flush=True)
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
           "--settle-ms", "0", "--sets", "1", "--no-cpu-baseline"] + mode
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.strip().splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    missing = KEYS - set(d)
    assert not missing, missing
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert "workload" in d["config"]
    rl = d["roofline"]
    assert 0 < rl["frac"] <= 1 and rl["peak"] > 0 and rl["achieved"] > 0


def test_bench_refuses_several_gpus():
    """More than one GPU is not part of this benchmark: the bench says so and exits."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "GPU" in (r.stderr + r.stdout)
