"""Helpers of the GPU parity tests: device copies of generated inputs, tolerance checks."""

import numpy as np
import torch

from bf16_hyper_connection_amd import hcr

TOL = 1e-4  # of the largest |value| of each output tensor (the pages' parity bound)


def dev():
    return torch.device("cuda:0")


def to_dev(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def reader_for(w):
    return hcr.HCRead(to_dev(w.w_down), to_dev(w.w_up), to_dev(w.w_norm))


def max_rel(got, ref):
    g = got.detach().double().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    scale = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(g - ref))) / (scale if scale > 0 else 1.0)


def check_read(reader, T, got_out, got_mean, ref, label, tol=TOL):
    """out, mean and lo within tol of the largest |value|; rs within 1e-5 per element."""
    torch.cuda.synchronize()
    lo, rs = reader.last_lo_rs(T)
    errs = {"out": max_rel(got_out, ref["out"]), "mean": max_rel(got_mean, ref["mean"]),
            "lo": max_rel(lo, ref["lo"])}
    rs_rel = float(np.max(np.abs(rs.double().cpu().numpy() / ref["rs"] - 1.0)))
    for k, e in errs.items():
        assert e <= tol, f"{label}: {k} error {e:.3e} > {tol:.0e} of max |ref|"
    assert rs_rel <= 1e-5, f"{label}: rs relative error {rs_rel:.3e}"
    return errs
