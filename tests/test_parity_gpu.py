"""Parity of the HIP read (through the C ABI) with the FP64 reference, on the GPU.

Every case runs at the real geometry (4 streams x 2560, R = 320) and compares
every element of out, mean and lo with the reference, within 1e-4 of the
largest |value| of each tensor (rs within 1e-5 relative).
"""

import numpy as np
import pytest
import torch

import oracle
from bf16_hyper_connection_amd import hcr
from bf16_hyper_connection_amd import inputs as gen
from tests import oracle_pins as pins
from tests.gpu_util import check_read, dev, reader_for, to_dev
from tests.libhcr_util import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


@pytest.fixture(scope="module")
def wset():
    w = gen.weight_set(1, 0)
    return w, reader_for(w)


def _read(reader, x, p, inj):
    out, mean = reader.read(to_dev(x), to_dev(p), to_dev(inj))
    return out, mean


@pytest.mark.parametrize("T", range(1, gen.T_WIDE + 1))
@pytest.mark.parametrize("with_pending", [False, True])
@pytest.mark.parametrize("with_inj", [False, True])
def test_matrix(wset, T, with_pending, with_inj):
    """T = 1..16 x pending write on/off x injection on/off (64 cases), one weight set."""
    w, reader = wset
    x = gen.activations(1, T, index=T)
    p = gen.pending(1, T, index=T) if with_pending else None
    inj = gen.injection(1, T, index=T) if with_inj else None
    out, mean = _read(reader, x, p, inj)
    ref = oracle.hc_read(x, w.w_norm, w.w_down, w.w_up, pending=p, inj=inj)
    check_read(reader, T, out, mean, ref, f"T={T} pending={with_pending} inj={with_inj}")


def test_single_read_seed0():
    """Real geometry, T = 1, one weight set, no pending write or injection (seed 0)."""
    c = gen.single_read(0)
    w = c["weights"][0]
    r = reader_for(w)
    out, mean = _read(r, c["x"], None, None)
    check_read(r, 1, out, mean, oracle.hc_read(c["x"], w.w_norm, w.w_down, w.w_up), "single read")


def test_full_epilogue_32_sets():
    """T = 4, pending write and injection on, 32 weight sets (seed 7)."""
    c = gen.full_epilogue(7)
    for k, w in enumerate(c["weights"]):
        r = reader_for(w)
        out, mean = _read(r, c["x"][k], c["pending"][k], c["inj"][k])
        ref = oracle.hc_read(c["x"][k], w.w_norm, w.w_down, w.w_up, pending=c["pending"][k], inj=c["inj"][k])
        check_read(r, 4, out, mean, ref, f"full epilogue set {k}")


def test_numerics_stress_32_sets():
    """T = 8, heavy-tailed x (stream RMS 1e-3..1e3), near-duplicate W_down rows, pending and inj on."""
    c = gen.numerics_stress(5)
    worst = 0.0
    for k, w in enumerate(c["weights"]):
        r = reader_for(w)
        out, mean = _read(r, c["x"][k], c["pending"][k], c["inj"][k])
        ref = oracle.hc_read(c["x"][k], w.w_norm, w.w_down, w.w_up, pending=c["pending"][k], inj=c["inj"][k])
        errs = check_read(r, 8, out, mean, ref, f"stress set {k}")
        worst = max(worst, max(errs.values()))
    print(f"numerics stress: worst error {worst:.3e} of max |ref|")


@pytest.mark.parametrize("T", [9, 12, 16])
def test_numerics_stress_wide_windows(T):
    """Windows beyond 8 tokens (two token groups in the down kernel) under the stress inputs, 4 weight sets."""
    c = gen.numerics_stress(6, T=T, n_sets=4)
    for k, w in enumerate(c["weights"]):
        r = reader_for(w)
        out, mean = _read(r, c["x"][k], c["pending"][k], c["inj"][k])
        ref = oracle.hc_read(c["x"][k], w.w_norm, w.w_down, w.w_up, pending=c["pending"][k], inj=c["inj"][k])
        check_read(r, T, out, mean, ref, f"wide stress T={T} set {k}")


def test_cold_rotation_all_sets_all_T():
    """The timed workload's launch pattern: 32 weight sets rotated per call, T = 1..8, each call checked."""
    ws = gen.cold_sweep_weights(32)
    readers = [reader_for(w) for w in ws]
    for T in range(1, 9):
        x = gen.cold_sweep_x(T)
        xd = to_dev(x)
        for k, (w, r) in enumerate(zip(ws, readers)):
            out, mean = r.read(xd)
            ref = oracle.hc_read(x, w.w_norm, w.w_down, w.w_up)
            check_read(r, T, out, mean, ref, f"rotation T={T} set {k}")


def test_closed_form_identity_weights():
    """Identity-like weights at the real geometry: the HIP read against the reference and the closed form."""
    (x, wn, wd, wu, p, inj), closed = pins.closed_form_case(4, 2560, 320, 3)
    w = gen.WeightSet(wd, wu, wn)
    r = reader_for(w)
    out, mean = _read(r, x, p, inj)
    ref = oracle.hc_read(x, wn, wd, wu, pending=p, inj=inj)
    check_read(r, 3, out, mean, ref, "closed form vs reference")
    check_read(r, 3, out, mean, closed, "closed form vs formula")


def test_zero_stream_and_saturated_gates(wset):
    w, reader = wset
    T = 5
    x = gen.activations(3, T)
    x[:, 1, :] = 0.0  # a zero stream: rs = 1000, no contribution
    inj = gen.injection(3, T)
    inj[:, 0] = 100.0   # gate of stream 0 open (sigmoid = 1)
    inj[:, 2] = -100.0  # gate of stream 2 shut (sigmoid ~ 0)
    p = gen.pending(3, T)
    out, mean = _read(reader, x, p, inj)
    ref = oracle.hc_read(x, w.w_norm, w.w_down, w.w_up, pending=p, inj=inj)
    check_read(reader, T, out, mean, ref, "zero stream / saturated gates")
    torch.cuda.synchronize()
    # the shut gate leaves the pending write (up to sigmoid(-100) * |u|)
    assert np.max(np.abs(out[:, 2].cpu().numpy() - p[:, 2])) <= 1e-30


def test_all_zero_input(wset):
    """x = 0 everywhere: rs = 1000, lo = inj = 0, out = pending + 0.5 * 0."""
    w, reader = wset
    T = 2
    x = np.zeros((T, 4, 2560), np.float32)
    p = gen.pending(4, T)
    out, mean = _read(reader, x, p, None)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), torch.from_numpy(p))
    lo, rs = reader.last_lo_rs(T)
    assert torch.all(lo == 0) and torch.allclose(rs.cpu(), torch.full((T, 4), 1000.0))


def test_empty_read_leaves_outputs(wset):
    """T = 0 enqueues nothing: non-empty out, mean and scratch filled with sentinels keep every byte."""
    _, reader = wset
    x = to_dev(gen.activations(3, 2))
    out = torch.full((2, 4, 2560), 7.0, device=dev())
    mean = torch.full((2, 2560), -3.0, device=dev())
    reader.scratch.fill_(0xA5)
    torch.cuda.synchronize()
    rc = hcr.hcr_read(reader.handle, 0, x.data_ptr(), None, None, out.data_ptr(), mean.data_ptr(),
                      torch.cuda.current_stream().cuda_stream)
    assert rc == hcr.HCR_OK
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(mean == -3.0) and torch.all(reader.scratch == 0xA5)
    # the binding's empty read is the same call
    reader.read(torch.empty((0, 4, 2560), device=dev()), out=torch.empty((0, 4, 2560), device=dev()),
                mean=torch.empty((0, 2560), device=dev()))
    torch.cuda.synchronize()
    assert torch.all(reader.scratch == 0xA5)


def test_in_place_out_on_x_and_on_pending(wset):
    w, reader = wset
    T = 6
    x = gen.activations(5, T)
    p = gen.pending(5, T)
    inj = gen.injection(5, T)
    ref_out, ref_mean = _read(reader, x, p, inj)
    xd = to_dev(x)
    out1, mean1 = reader.read(xd, to_dev(p), to_dev(inj), out=xd)
    pd = to_dev(p)
    out2, mean2 = reader.read(to_dev(x), pd, to_dev(inj), out=pd)
    torch.cuda.synchronize()
    assert out1.data_ptr() == xd.data_ptr() and out2.data_ptr() == pd.data_ptr()
    for o, m in ((out1, mean1), (out2, mean2)):
        assert torch.equal(o, ref_out) and torch.equal(m, ref_mean)


def test_repeated_reads_bitwise(wset):
    w, reader = wset
    T = 7
    xd, pd, idd = to_dev(gen.activations(6, T)), to_dev(gen.pending(6, T)), to_dev(gen.injection(6, T))
    o0, m0 = reader.read(xd, pd, idd)
    o0, m0 = o0.clone(), m0.clone()
    for _ in range(100):
        o, m = reader.read(xd, pd, idd)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(m, m0)


def test_distinct_handles_on_two_streams():
    """Two handles (two weight sets, each with its own scratch) reading at the same time on two streams:
    every result equals the same read made alone, bit for bit."""
    sets = [gen.weight_set(30, k) for k in range(2)]
    readers = [reader_for(w) for w in sets]
    T = (5, 12)
    xs = [to_dev(gen.activations(31, T[k], index=k)) for k in range(2)]
    ps = [to_dev(gen.pending(31, T[k], index=k)) for k in range(2)]
    ij = [to_dev(gen.injection(31, T[k], index=k)) for k in range(2)]
    alone = []
    for k in range(2):
        o, m = readers[k].read(xs[k], ps[k], ij[k])
        torch.cuda.synchronize()
        alone.append((o.clone(), m.clone()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    outs = [[None] * 2 for _ in range(20)]
    for i in range(20):
        for k in range(2):
            with torch.cuda.stream(streams[k]):
                outs[i][k] = readers[k].read(xs[k], ps[k], ij[k])
    torch.cuda.synchronize()
    for i in range(20):
        for k in range(2):
            o, m = outs[i][k]
            assert torch.equal(o, alone[k][0]) and torch.equal(m, alone[k][1]), f"round {i} handle {k}"


@pytest.mark.parametrize("lo_t,hi_t,windows", [
    (1, 8, [(0, 1), (5, 6), (7, 8), (0, 2), (3, 5), (6, 8), (1, 4), (2, 7), (0, 7), (1, 8), (4, 7)]),
    (9, 16, [(0, 9), (7, 16), (0, 10), (6, 16), (2, 15), (3, 14), (1, 13), (4, 16)]),
])
def test_token_results_do_not_depend_on_T(wset, lo_t, hi_t, windows):
    """Each of the matrix-core kernel's B layouts (T = 1..8: high and low parts side by side; T = 9..16: one
    B matrix per part) gives each token the same result, bit for bit, in every window of its range (a token
    read alone included)."""
    w, reader = wset
    T = hi_t
    x, p, inj = gen.activations(8 + T, T), gen.pending(8 + T, T), gen.injection(8 + T, T)
    ofull, mfull = _read(reader, x, p, inj)
    ofull, mfull = ofull.clone(), mfull.clone()
    for a, b in windows:
        assert lo_t <= b - a < hi_t
        o, m = _read(reader, x[a:b], p[a:b], inj[a:b])
        torch.cuda.synchronize()
        assert torch.equal(o, ofull[a:b]) and torch.equal(m, mfull[a:b]), f"tokens {a}..{b - 1}"


def test_single_token_reads_equal_the_window(wset):
    """Every token of an 8-token window read alone (T = 1) gives the window's out and mean for it, bit for bit:
    both run the matrix-core up kernel with the same B layout."""
    w, reader = wset
    T = 8
    x, p, inj = gen.activations(19, T), gen.pending(19, T), gen.injection(19, T)
    o8, m8 = _read(reader, x, p, inj)
    o8, m8 = o8.clone(), m8.clone()
    for t in range(T):
        o1, m1 = _read(reader, x[t:t + 1], p[t:t + 1], inj[t:t + 1])
        torch.cuda.synchronize()
        assert torch.equal(o1[0], o8[t]) and torch.equal(m1[0], m8[t]), f"token {t}"


def test_numerics_stress_graph_replay_bitwise():
    """The stress workload's 32 reads captured in one graph: replays equal the direct calls bit for bit."""
    c = gen.numerics_stress(5, n_sets=32)
    readers = [reader_for(w) for w in c["weights"]]
    xs = [to_dev(x) for x in c["x"]]
    ps = [to_dev(p) for p in c["pending"]]
    ij = [to_dev(i) for i in c["inj"]]
    outs = [torch.empty((8, 4, 2560), device=dev()) for _ in readers]
    means = [torch.empty((8, 2560), device=dev()) for _ in readers]
    for k, r in enumerate(readers):
        r.read(xs[k], ps[k], ij[k], out=outs[k], mean=means[k])
    torch.cuda.synchronize()
    direct = [(o.clone(), m.clone()) for o, m in zip(outs, means)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for k, r in enumerate(readers):
                r.read(xs[k], ps[k], ij[k], out=outs[k], mean=means[k])
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for o, m in zip(outs, means):
            o.fill_(float("nan"))
            m.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for k, (o, m) in enumerate(direct):
            assert torch.equal(outs[k], o) and torch.equal(means[k], m), f"replay {rep} read {k}"


@pytest.mark.parametrize("T", [1, 6, 8, 9, 16])
def test_graph_replay_bitwise(wset, T):
    """A captured read replayed several times (with eager work between) equals the direct call, bitwise."""
    w, reader = wset
    xd, pd, idd = to_dev(gen.activations(9, T)), to_dev(gen.pending(9, T)), to_dev(gen.injection(9, T))
    direct_o, direct_m = reader.read(xd, pd, idd)
    direct_o, direct_m = direct_o.clone(), direct_m.clone()
    out = torch.empty_like(direct_o)
    mean = torch.empty_like(direct_m)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            reader.read(xd, pd, idd, out=out, mean=mean)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(4):
        out.fill_(float("nan"))
        mean.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, direct_o) and torch.equal(mean, direct_m), f"replay {i}"
        # eager work between replays, on other buffers
        reader.read(to_dev(gen.activations(10 + i, T)))
        torch.cuda.synchronize()
