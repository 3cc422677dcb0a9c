"""Q8_0 copies on the GPU (through the C ABI) against the FP64 reference.

The quantiser is integer/byte work: codes and binary16 scale patterns must be
bitwise equal to the reference's.  The read on the copies is compared element
by element with the reference read on the reference's own copies, within
1e-4 of the largest |value| of each tensor, like the BF16 read.
"""

import numpy as np
import pytest
import torch

import oracle
from bf16_hyper_connection_amd import hcr
from bf16_hyper_connection_amd import inputs as gen
from tests.gpu_util import check_read, dev, to_dev
from tests.libhcr_util import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _quantize_on_gpu(bits):
    codes, scales = hcr.quantize_q8_0(to_dev(bits))
    torch.cuda.synchronize()
    return codes, scales


def _assert_same_copy(bits, label):
    codes, scales = _quantize_on_gpu(bits)
    ref_codes, ref_scales = oracle.quantize_q8_0(bits)
    got_c = codes.cpu().numpy()
    got_s = scales.cpu().numpy().view(np.uint16)
    bad_c = np.count_nonzero(got_c != ref_codes)
    bad_s = np.count_nonzero(got_s != ref_scales)
    assert bad_c == 0 and bad_s == 0, f"{label}: {bad_c} codes and {bad_s} scales differ"
    return codes, scales


def test_quantize_edge_blocks_bitwise():
    """Every edge family (zeros, ties, tiny / subnormal / overflowing scales, negative maxima) bit for bit."""
    _assert_same_copy(gen.q8_edge_weights(3), "edge blocks")
    _assert_same_copy(gen.q8_edge_weights(4, rows=7, K=352), "edge blocks, ragged grid")


@pytest.mark.parametrize("k", [0, 1])
def test_quantize_read_weights_bitwise(k):
    """The read's real matrices: W_down [320][10240] and W_up [10240][320]."""
    w = gen.weight_set(12, k)
    _assert_same_copy(w.w_down, f"W_down set {k}")
    _assert_same_copy(w.w_up, f"W_up set {k}")


def test_quantize_single_block():
    """One block (a grid of one partly filled work-group)."""
    _assert_same_copy(gen.q8_edge_weights(6, rows=1, K=32), "single block")


class Q8Set:
    """A weight set's Q8_0 copies made on the GPU, and the reference's copies."""

    def __init__(self, w):
        self.w = w
        dc, ds = _quantize_on_gpu(w.w_down)
        uc, us = _quantize_on_gpu(w.w_up)
        self.reader = hcr.HCRead.q8_0(dc, ds, uc, us, to_dev(w.w_norm))
        self.ref_down = oracle.quantize_q8_0(w.w_down)
        self.ref_up = oracle.quantize_q8_0(w.w_up)

    def ref_read(self, x, p=None, inj=None):
        return oracle.hc_read_q8_0(x, self.w.w_norm, *self.ref_down, *self.ref_up, pending=p, inj=inj)


@pytest.fixture(scope="module")
def q8set():
    return Q8Set(gen.weight_set(13, 0))


@pytest.mark.parametrize("T", range(1, 9))
@pytest.mark.parametrize("with_pending", [False, True])
@pytest.mark.parametrize("with_inj", [False, True])
def test_q8_matrix(q8set, T, with_pending, with_inj):
    """T = 1..8 x pending on/off x injection on/off on the Q8_0 copies."""
    x = gen.activations(13, T, index=T)
    p = gen.pending(13, T, index=T) if with_pending else None
    inj = gen.injection(13, T, index=T) if with_inj else None
    out, mean = q8set.reader.read(to_dev(x), to_dev(p), to_dev(inj))
    check_read(q8set.reader, T, out, mean, q8set.ref_read(x, p, inj), f"Q8_0 T={T} p={with_pending} i={with_inj}")


@pytest.mark.parametrize("T", range(9, gen.T_WIDE + 1))
def test_q8_wide_windows(q8set, T):
    x, p, inj = gen.activations(14, T, index=T), gen.pending(14, T, index=T), gen.injection(14, T, index=T)
    out, mean = q8set.reader.read(to_dev(x), to_dev(p), to_dev(inj))
    check_read(q8set.reader, T, out, mean, q8set.ref_read(x, p, inj), f"Q8_0 T={T}")


@pytest.mark.parametrize("T", [9, 12, 16])
@pytest.mark.parametrize("with_pending,with_inj", [(False, False), (False, True), (True, False)])
def test_q8_wide_windows_epilogue_variants(q8set, T, with_pending, with_inj):
    """The matrix-core kernels of the larger windows (3 waves at T = 9, 4 from T = 10) without the pending write
    or the injection."""
    x = gen.activations(24, T, index=T)
    p = gen.pending(24, T, index=T) if with_pending else None
    inj = gen.injection(24, T, index=T) if with_inj else None
    out, mean = q8set.reader.read(to_dev(x), to_dev(p), to_dev(inj))
    check_read(q8set.reader, T, out, mean, q8set.ref_read(x, p, inj), f"Q8_0 T={T} p={with_pending} i={with_inj}")


@pytest.mark.parametrize("T", [2, 3, 8])
def test_q8_numerics_stress(T):
    """Heavy-tailed x (stream RMS 1e-3..1e3), near-duplicate W_down rows, pending and inj, 4 sets; T = 2 and 3
    sit on either side of the switch from the vector-ALU to the matrix-core up kernel."""
    c = gen.numerics_stress(15, T=T, n_sets=4)
    for k, w in enumerate(c["weights"]):
        s = Q8Set(w)
        out, mean = s.reader.read(to_dev(c["x"][k]), to_dev(c["pending"][k]), to_dev(c["inj"][k]))
        check_read(s.reader, T, out, mean, s.ref_read(c["x"][k], c["pending"][k], c["inj"][k]),
                   f"Q8_0 stress T={T} set {k}")


@pytest.mark.parametrize("lo_t,hi_t,windows", [
    (1, 2, [(0, 1), (1, 2), (0, 2)]),
    (3, 8, [(0, 3), (5, 8), (0, 4), (4, 8), (1, 6), (2, 8), (0, 7), (1, 8)]),
    (9, 16, [(0, 9), (7, 16), (2, 13), (3, 15), (0, 15), (1, 16)]),
])
def test_q8_token_results_do_not_depend_on_T(q8set, lo_t, hi_t, windows):
    """Q8_0 reads: within each range of T that one up kernel serves (T = 1..2 vector ALUs; T = 3..8 and
    9..16 the matrix cores' two B layouts) each token's result is the same, bit for bit, in every window."""
    T = hi_t
    x, p, inj = gen.activations(16 + T, T), gen.pending(16 + T, T), gen.injection(16 + T, T)
    of, mf = q8set.reader.read(to_dev(x), to_dev(p), to_dev(inj))
    of, mf = of.clone(), mf.clone()
    for a, b in windows:
        assert lo_t <= b - a <= hi_t
        o, m = q8set.reader.read(to_dev(x[a:b]), to_dev(p[a:b]), to_dev(inj[a:b]))
        torch.cuda.synchronize()
        assert torch.equal(o, of[a:b]) and torch.equal(m, mf[a:b]), f"tokens {a}..{b - 1}"


@pytest.mark.parametrize("T", [1, 2, 3, 8, 9, 16])
def test_q8_graph_replay_bitwise(q8set, T):
    r = q8set.reader
    xd, pd, idd = to_dev(gen.activations(17, T)), to_dev(gen.pending(17, T)), to_dev(gen.injection(17, T))
    direct_o, direct_m = r.read(xd, pd, idd)
    direct_o, direct_m = direct_o.clone(), direct_m.clone()
    out, mean = torch.empty_like(direct_o), torch.empty_like(direct_m)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            r.read(xd, pd, idd, out=out, mean=mean)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(4):
        out.fill_(float("nan"))
        mean.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, direct_o) and torch.equal(mean, direct_m), f"replay {i}"


def test_q8_quantize_in_a_graph_bitwise():
    """The quantiser captured in a graph and replayed equals the direct call."""
    w = to_dev(gen.weight_set(18, 0).w_up)
    c0, s0 = hcr.quantize_q8_0(w)
    c0, s0 = c0.clone(), s0.clone()
    codes, scales = torch.empty_like(c0), torch.empty_like(s0)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            rc = hcr.hcr_quantize_q8_0(w.data_ptr(), w.shape[0], w.shape[1], codes.data_ptr(), scales.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream)
            assert rc == hcr.HCR_OK
    torch.cuda.current_stream().wait_stream(st)
    for i in range(3):
        codes.fill_(0)
        scales.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(codes, c0) and torch.equal(scales, s0), f"replay {i}"


def test_q8_residual_chain_of_16_reads():
    """A verify-window chain on Q8_0 copies: 16 reads, out_i = x_{i+1}, T = 6, pending on; each step against the
    reference on the x the GPU fed it."""
    n, T = 16, 6
    c = gen.verify_window(n, T, base=19)
    sets = [Q8Set(w) for w in c["weights"]]
    x = to_dev(c["x0"])
    x_host = c["x0"]
    for i, s in enumerate(sets):
        out, mean = s.reader.read(x, to_dev(c["pending"][i]))
        torch.cuda.synchronize()
        ref = s.ref_read(x_host, c["pending"][i])
        check_read(s.reader, T, out, mean, ref, f"Q8_0 chain step {i}")
        x, x_host = out, out.cpu().numpy()


def test_quantize_overflowing_block_scale_is_infinite_and_read_is_not_finite():
    """A block whose largest |w| exceeds 127 * 65504 (the largest finite binary16 times 127) gets d = amax / 127
    above binary16's range: the stored scale is +inf (as the reference's), and a read on such copies has
    non-finite outputs.  The header states the bound; the weights of the read here stay far below it."""
    w = gen.weight_set(13, 0)
    bits = w.w_down.copy()
    big = np.float32(2.0e7)  # its BF16 truncation is still far above 127 * 65504 = 8,319,008
    b16 = (np.array([big], np.float32).view(np.uint32) >> 16).astype(np.uint16)[0]
    bits[5, 64] = b16  # row 5, block 2
    codes, scales = _assert_same_copy(bits, "one overflowing block")
    s = scales.cpu().numpy().view(np.uint16)
    assert s[5, 2] == 0x7C00, hex(int(s[5, 2]))          # +inf in binary16
    assert np.all(s[5, :2] != 0x7C00) and np.all(s[4] != 0x7C00)
    uc, us = _quantize_on_gpu(w.w_up)
    reader = hcr.HCRead.q8_0(codes, scales, uc, us, to_dev(w.w_norm))
    out, mean = reader.read(to_dev(gen.activations(13, 2)))
    torch.cuda.synchronize()
    assert not torch.isfinite(out).all() and not torch.isfinite(mean).all()
