"""hcr_read_static, the read on the library's own device scratch (no handle, no caller scratch, no
allocation), against hcr_read on a handle of the same weights: two calls in a row, the second with fewer
tokens, both bitwise equal to the handle's reads and within the tolerance of the FP64 reference."""

import numpy as np
import pytest
import torch

import oracle
from bf16_hyper_connection_amd import hcr
from bf16_hyper_connection_amd import inputs as gen
from tests.gpu_util import TOL, dev, max_rel, reader_for, to_dev
from tests.libhcr_util import ensure_built

pytestmark = pytest.mark.gpu


def _static(w_dev, T, x, p, inj, out, mean):
    st = torch.cuda.current_stream().cuda_stream
    rc = hcr.hcr_read_static(w_dev[0].data_ptr(), w_dev[1].data_ptr(), w_dev[2].data_ptr(), T, x.data_ptr(),
                             None if p is None else p.data_ptr(), None if inj is None else inj.data_ptr(),
                             out.data_ptr(), mean.data_ptr(), st)
    assert rc == hcr.HCR_OK, hcr.hcr_strerror(rc)


@pytest.mark.parametrize("Ts", [(8, 3), (16, 1), (6, 2)])
def test_read_static_equals_handle_read(Ts):
    ensure_built()
    w = gen.weight_set(40, Ts[0])
    reader = reader_for(w)
    w_dev = (reader.w_down, reader.w_up, reader.w_norm)
    for k, T in enumerate(Ts):
        print(f"hcr_read_static: call {k}, T={T}", flush=True)
        x, p, inj = gen.activations(41 + k, T), gen.pending(41 + k, T), gen.injection(41 + k, T)
        xd, pd, idd = to_dev(x), to_dev(p), to_dev(inj)
        out = torch.full((T, 4, 2560), float("nan"), device=dev())
        mean = torch.full((T, 2560), float("nan"), device=dev())
        _static(w_dev, T, xd, pd, idd, out, mean)
        ref_o, ref_m = reader.read(xd, pd, idd)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(mean, ref_m), f"call {k} (T={T}) differs from hcr_read"
        ref = oracle.hc_read(x, w.w_norm, w.w_down, w.w_up, pending=p, inj=inj)
        assert max_rel(out, ref["out"]) <= TOL and max_rel(mean, ref["mean"]) <= TOL


def test_read_static_in_a_graph_with_eager_work_between():
    """Captured (no allocation inside), replayed with eager reads between: every replay equals the direct call."""
    ensure_built()
    w = gen.weight_set(42, 0)
    reader = reader_for(w)
    w_dev = (reader.w_down, reader.w_up, reader.w_norm)
    T = 5
    xd = to_dev(gen.activations(43, T))
    out = torch.empty((T, 4, 2560), device=dev())
    mean = torch.empty((T, 2560), device=dev())
    _static(w_dev, T, xd, None, None, out, mean)
    torch.cuda.synchronize()
    direct_o, direct_m = out.clone(), mean.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            rc = hcr.hcr_read_static(w_dev[0].data_ptr(), w_dev[1].data_ptr(), w_dev[2].data_ptr(), T, xd.data_ptr(),
                                     None, None, out.data_ptr(), mean.data_ptr(), s.cuda_stream)
            assert rc == hcr.HCR_OK
    torch.cuda.current_stream().wait_stream(s)
    for i in range(3):
        out.fill_(float("nan"))
        mean.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, direct_o) and torch.equal(mean, direct_m), f"replay {i}"
        o2 = torch.empty((2, 4, 2560), device=dev())
        m2 = torch.empty((2, 2560), device=dev())
        _static(w_dev, 2, to_dev(gen.activations(44 + i, 2)), None, None, o2, m2)  # eager, smaller, same array
        torch.cuda.synchronize()
    assert np.isfinite(direct_o.cpu().numpy()).all()
