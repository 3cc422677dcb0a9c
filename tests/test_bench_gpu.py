"""bench.py's output line on the GPU: one JSON object with the fields and units the measurement reports, and
figures that agree with each other (µs per read from ms per step, the roofline fraction from achieved / peak,
the counter traffic of the current sources).  bench.py runs as a child process on a short setting."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_line_fields_and_consistency():
    args = [sys.executable, "bench.py", "--steps", "3", "--warmup", "1", "--per-t-reps", "1", "--no-window",
            "--no-q8", "--no-matvec", "--no-cpu-baseline"]
    print("bench child:", " ".join(args[1:]), flush=True)
    r = subprocess.run(args, capture_output=True, text=True, cwd=ROOT, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    b = json.loads(lines[0])

    assert b["unit"] == "µs" and b["higher_is_better"] is False and b["n_gpus"] == 1
    assert b["steps"] == 3 and b["warmup"] == 1 and b["vs_baseline"] is None
    assert b["dtype"] == "bf16" and b["data"] == "synthetic" and b["scaling"] == "weak"
    cfg = b["config"]
    assert cfg["workload"] and "model" not in cfg
    assert cfg["weight_sets"] == 32 and cfg["reads_per_step"] == 8 * 32
    assert sorted(int(t) for t in cfg["per_T_us"]) == list(range(1, 9))

    # µs per read is the step time over the step's reads
    assert b["value"] > 0
    assert abs(b["value"] - b["ms_per_step"] * 1000.0 / cfg["reads_per_step"]) <= 0.002 + 1e-3 * b["value"]

    rl = b["roofline"]
    assert rl["bound"] == "hbm" and rl["unit"] == "GB/s" and rl["peak"] == 8000.0
    assert 0 < rl["frac"] < 1 and abs(rl["frac"] - rl["achieved"] / rl["peak"]) <= 1e-4
    # achieved = algorithmic bytes per read (mean over T = 1..8, no pending write or injection) / µs per read
    alg = sum(13_107_200 + 40_960 + T * 92_160 for T in range(1, 9)) / 8
    assert abs(rl["achieved"] - alg / (b["value"] * 1e3)) <= 0.01 * rl["achieved"]
    # the counter record is keyed to the library sources: null once the kernels change, else bytes per read
    assert rl["traffic"] is None or (isinstance(rl["traffic"], int) and alg < rl["traffic"] < 1.2 * alg)
    assert "cpu_baseline" not in b
