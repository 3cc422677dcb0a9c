"""The C ABI from plain C: tests/c_caller/hcr_read_file.c includes only include/hcr.h and the HIP
runtime's C header, allocates with hipMalloc and calls the library's entry points, with no Python
or torch in the process.  The CPU tests check that it builds as strict C11 and rejects bad
arguments; the GPU tests run it as a child process on seeded inputs written to files and compare
what it writes with the FP64 oracle."""

import os
import subprocess

import numpy as np
import pytest

import oracle
from bf16_hyper_connection_amd import build
from bf16_hyper_connection_amd import inputs as gen
from tests.libhcr_util import ensure_built

TOL = 1e-4  # of the largest |value| of each output tensor, as in the other parity tests


@pytest.fixture(scope="module")
def caller():
    ensure_built()
    if not os.path.exists(build.C_CALLER):
        build.build_c_caller()
    return build.C_CALLER


def _run(caller, *args, timeout=60):
    return subprocess.run([caller] + [str(a) for a in args], capture_output=True, text=True, timeout=timeout)


@pytest.mark.parametrize("args,msg", [
    ((), "usage"),
    (("/nonexistent", 0), "T"),
    (("/nonexistent", 17), "T"),
    (("/nonexistent", 2, "bogus"), "unknown option"),
])
def test_rejects_bad_arguments_before_any_device_work(caller, args, msg):
    res = _run(caller, *args)
    assert res.returncode == 1 and msg in res.stderr, res.stderr


def _write_inputs(d, w, x, p, inj):
    w.w_down.tofile(os.path.join(d, "w_down.bin"))
    w.w_up.tofile(os.path.join(d, "w_up.bin"))
    w.w_norm.astype(np.float32).tofile(os.path.join(d, "w_norm.bin"))
    x.astype(np.float32).tofile(os.path.join(d, "x.bin"))
    if p is not None:
        p.astype(np.float32).tofile(os.path.join(d, "pending.bin"))
    if inj is not None:
        inj.astype(np.float32).tofile(os.path.join(d, "inj.bin"))


def _check(d, T, ref, label):
    S, D = gen.S_STREAMS, gen.D_STREAM
    got = {"out": np.fromfile(os.path.join(d, "out.bin"), np.float32).reshape(T, S, D),
           "mean": np.fromfile(os.path.join(d, "mean.bin"), np.float32).reshape(T, D)}
    for name, g in got.items():
        err = np.max(np.abs(g.astype(np.float64) - ref[name])) / np.max(np.abs(ref[name]))
        assert err <= TOL, f"{label}: {name} error {err:.3e} > {TOL:.0e} of max |ref|"


@pytest.mark.gpu
@pytest.mark.parametrize("T,with_pending,with_inj", [(1, False, False), (3, True, True), (16, True, False)])
def test_bf16_read_from_c(caller, tmp_path, T, with_pending, with_inj):
    w = gen.weight_set(40, 0)
    x = gen.activations(40, T)
    p = gen.pending(40, T) if with_pending else None
    inj = gen.injection(40, T) if with_inj else None
    _write_inputs(tmp_path, w, x, p, inj)
    args = [tmp_path, T] + (["pending"] if with_pending else []) + (["inj"] if with_inj else [])
    print(f"C caller: BF16 T={T} pending={with_pending} inj={with_inj}", flush=True)
    res = _run(caller, *args)
    assert res.returncode == 0, res.stderr
    ref = oracle.hc_read(x, w.w_norm, w.w_down, w.w_up, pending=p, inj=inj)
    _check(tmp_path, T, ref, f"C caller BF16 T={T}")


@pytest.mark.gpu
def test_q8_0_read_from_c(caller, tmp_path):
    """The C caller quantises both projections with hcr_quantize_q8_0 and reads the copies."""
    T = 2
    w = gen.weight_set(41, 0)
    x = gen.activations(41, T)
    inj = gen.injection(41, T)
    _write_inputs(tmp_path, w, x, None, inj)
    print("C caller: Q8_0 T=2 inj", flush=True)
    res = _run(caller, tmp_path, T, "inj", "q8")
    assert res.returncode == 0, res.stderr
    ref = oracle.hc_read_q8_0(x, w.w_norm, *oracle.quantize_q8_0(w.w_down), *oracle.quantize_q8_0(w.w_up),
                              inj=inj)
    _check(tmp_path, T, ref, "C caller Q8_0 T=2")
