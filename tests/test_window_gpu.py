"""The 96-read verify window on the GPU: a residual chain (out_i is x_{i+1}) over 96 distinct
weight sets at T = 6 with the pending write on, captured as one HIP graph.

Each step is graded against the FP64 reference on the x the GPU actually fed it (the chain's
FP32 rounding compounds, so the whole-chain FP64 drift is reported, not graded), and graph
replays must equal the direct chain bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
from bf16_hyper_connection_amd import inputs as gen
from tests.gpu_util import TOL, dev, max_rel, reader_for, to_dev
from tests.libhcr_util import ensure_built

pytestmark = pytest.mark.gpu

N_READS, T = 96, 6


@pytest.fixture(scope="module")
def window():
    ensure_built()
    c = gen.verify_window(N_READS, T)
    readers = [reader_for(w) for w in c["weights"]]
    pend = [to_dev(p) for p in c["pending"]]
    x0 = to_dev(c["x0"])
    return c, readers, pend, x0


def _chain(readers, pend, x0, outs, means):
    x = x0
    for i, r in enumerate(readers):
        r.read(x, pend[i], None, out=outs[i], mean=means[i])
        x = outs[i]


def test_window_steps_and_graph_replay(window):
    c, readers, pend, x0 = window
    outs = [torch.empty((T, 4, 2560), device=dev()) for _ in range(N_READS)]
    means = [torch.empty((T, 2560), device=dev()) for _ in range(N_READS)]
    _chain(readers, pend, x0, outs, means)
    torch.cuda.synchronize()
    direct_o = [o.clone() for o in outs]
    direct_m = [m.clone() for m in means]

    # every step against the reference, on the x the GPU saw
    worst = 0.0
    x_prev = c["x0"]
    for i, w in enumerate(c["weights"]):
        ref = oracle.hc_read(x_prev, w.w_norm, w.w_down, w.w_up, pending=c["pending"][i])
        e = max(max_rel(direct_o[i], ref["out"]), max_rel(direct_m[i], ref["mean"]))
        assert e <= TOL, f"window step {i}: error {e:.3e}"
        worst = max(worst, e)
        x_prev = direct_o[i].cpu().numpy()
    print(f"window: worst per-step error {worst:.3e} of max |ref|")

    # one graph of the 96 reads, replayed with eager work in between
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            _chain(readers, pend, x0, outs, means)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for o, m in zip(outs, means):
            o.fill_(float("nan"))
            m.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i in range(N_READS):
            assert torch.equal(outs[i], direct_o[i]) and torch.equal(means[i], direct_m[i]), f"replay {rep} step {i}"
        readers[0].read(to_dev(gen.activations(11, T)))  # eager work between replays
        torch.cuda.synchronize()


def test_window_drift_of_the_fp64_chain(window):
    """Reported, not graded: the FP64 chain run end to end vs the GPU chain."""
    c, readers, pend, x0 = window
    outs = [torch.empty((T, 4, 2560), device=dev()) for _ in range(N_READS)]
    means = [torch.empty((T, 2560), device=dev()) for _ in range(N_READS)]
    _chain(readers, pend, x0, outs, means)
    torch.cuda.synchronize()
    x = c["x0"].astype(np.float64)
    for i, w in enumerate(c["weights"]):
        x = oracle.hc_read(x, w.w_norm, w.w_down, w.w_up, pending=c["pending"][i])["out"]
    drift = max_rel(outs[-1], x)
    print(f"window: FP64 end-to-end drift after {N_READS} reads {drift:.3e} of max |ref|")
    assert np.isfinite(drift)
