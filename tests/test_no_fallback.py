"""The product has no CPU path: bench.py, smoke() and the binding fail loudly where the GPU or the built library
is missing, and bench.py refuses more than one GPU.  Each case runs in a child process (no GPU is touched)."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(code_or_args, timeout=300):
    args = [sys.executable] + (["-c", code_or_args] if isinstance(code_or_args, str) else code_or_args)
    return subprocess.run(args, capture_output=True, text=True, cwd=ROOT, timeout=timeout)


def _gpu_visible():
    r = _run("import torch; print(torch.cuda.device_count())", timeout=600)
    return r.returncode == 0 and r.stdout.strip() not in ("", "0")


def test_bench_refuses_more_than_one_gpu():
    r = _run(["bench.py", "--gpus", "2"])
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_missing_library_raises():
    """With libhcr.so absent, the binding raises instead of computing anything another way."""
    code = ("import bf16_hyper_connection_amd.hcr as h\n"
            "h.LIB_PATH = '/nonexistent/libhcr.so'\n"
            "try:\n"
            "    h.lib()\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n")
    r = _run(code)
    assert r.returncode == 0 and "raised:" in r.stdout and "missing" in r.stdout


@pytest.mark.skipif(_gpu_visible(), reason="checks the behaviour where no GPU is visible")
def test_bench_and_smoke_fail_without_a_gpu():
    r = _run(["bench.py", "--steps", "1", "--warmup", "0", "--no-cpu-baseline", "--no-window", "--no-q8",
              "--no-matvec"])
    assert r.returncode != 0 and "GPU" in r.stderr
    r = _run("import __graft_entry__ as g\ng.smoke()")
    assert r.returncode != 0 and "GPU" in r.stderr
