"""libhcr_calib.so (include/hcr_calib.h), the calibration kernels of bench.py: it loads, exports what its
header declares and rejects bad arguments before any HIP call (CPU); on the GPU both pairs run."""

import ctypes
import os
import re

import pytest

from bf16_hyper_connection_amd import build
from tests.libhcr_util import ROOT, ensure_built

HEADER = os.path.join(ROOT, "include", "hcr_calib.h")
HCR_OK, HCR_EINVAL, HCR_EALIGN = 0, -1, -2


@pytest.fixture(scope="module")
def cal():
    ensure_built()
    if not os.path.exists(build.CALIB_LIB):
        build.build()
    L = ctypes.CDLL(build.CALIB_LIB)
    vp = ctypes.c_void_p
    L.hcrc_read_floor.restype = ctypes.c_int
    L.hcrc_read_floor.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp]
    L.hcrc_up_kernel.restype = ctypes.c_int
    L.hcrc_up_kernel.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp]
    L.hcrc_slab_pair.restype = ctypes.c_int
    L.hcrc_slab_pair.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp]
    L.hcrc_slab_read.restype = ctypes.c_int
    L.hcrc_slab_read.argtypes = [ctypes.c_int] + [vp] * 10
    return L


def test_exports_every_declared_symbol(cal):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(hcrc_[a-z_]+)\s*\(", text)))
    assert names == ["hcrc_read_floor", "hcrc_slab_pair", "hcrc_slab_read", "hcrc_up_kernel"]
    for n in names:
        assert hasattr(cal, n)


FAKE = dict(wd=0x10000000, wu=0x20000000, wn=0x30000000, sc=0x40000000, x=0x50000000)


@pytest.mark.parametrize("kind,T,kw,rc", [
    (3, 1, {}, HCR_EINVAL),            # unknown kind
    (-1, 1, {}, HCR_EINVAL),
    (0, 0, {}, HCR_EINVAL),            # T out of range
    (1, 17, {}, HCR_EINVAL),
    (1, 1, dict(wd=None), HCR_EINVAL),
    (1, 1, dict(x=None), HCR_EINVAL),
    (1, 1, dict(sc=None), HCR_EINVAL),
    (1, 1, dict(wu=0x20000008), HCR_EALIGN),
    (1, 1, dict(sc=0x40000010), HCR_EALIGN),
    (1, 1, dict(x=0x50000004), HCR_EALIGN),
])
def test_rejects_before_any_hip_call(cal, kind, T, kw, rc):
    a = dict(FAKE)
    a.update(kw)
    assert cal.hcrc_read_floor(kind, T, a["wd"], a["wu"], a["wn"], a["sc"], a["x"], None) == rc


@pytest.mark.gpu
@pytest.mark.parametrize("T", [1, 2, 8, 9, 10, 16])
def test_pairs_run_and_write_nothing(cal, T):
    import numpy as np
    import torch

    from bf16_hyper_connection_amd import hcr
    from bf16_hyper_connection_amd import inputs as gen
    from tests.gpu_util import reader_for, to_dev

    print(f"calibration pairs T={T}", flush=True)
    r = reader_for(gen.weight_set(0, 0))
    x = to_dev(gen.activations(0, T))
    snap = [t.clone() for t in (r.w_down, r.w_up, r.w_norm, r.scratch, x)]
    st = torch.cuda.current_stream().cuda_stream
    for kind in (0, 1):
        rc = cal.hcrc_read_floor(kind, T, r.w_down.data_ptr(), r.w_up.data_ptr(), r.w_norm.data_ptr(),
                                 r.scratch.data_ptr(), x.data_ptr(), st)
        assert rc == HCR_OK, hcr.hcr_strerror(rc)
    torch.cuda.synchronize()
    for a, b in zip(snap, (r.w_down, r.w_up, r.w_norm, r.scratch, x)):
        assert torch.equal(a, b)
    # HCRC_LOADS_STORE writes one float per down work-group into the lo slot, nothing else
    rc = cal.hcrc_read_floor(2, T, r.w_down.data_ptr(), r.w_up.data_ptr(), r.w_norm.data_ptr(), r.scratch.data_ptr(),
                             x.data_ptr(), st)
    assert rc == HCR_OK
    torch.cuda.synchronize()
    lo_off = hcr.hcr_scratch_layout()[0]
    f = r.scratch.view(torch.float32)
    assert torch.all(f[lo_off // 4: lo_off // 4 + 256] == 1.0)
    assert torch.equal(r.scratch[:lo_off], snap[3][:lo_off]) and torch.equal(r.scratch[lo_off + 1024:], snap[3][lo_off + 1024:])
    assert np.isfinite(x.cpu().numpy()).all()


@pytest.mark.parametrize("kind,T,kw,rc", [
    (2, 1, {}, HCR_EINVAL),
    (0, 0, {}, HCR_EINVAL),
    (1, 17, {}, HCR_EINVAL),
    (1, 2, dict(out=None), HCR_EINVAL),
    (0, 2, dict(sc=None), HCR_EINVAL),
    (1, 2, dict(sc=0x40000040), HCR_EALIGN),
    (0, 2, dict(mean=0x70000004), HCR_EALIGN),
])
def test_up_kernel_rejects_before_any_hip_call(cal, kind, T, kw, rc):
    a = dict(wu=0x20000000, sc=0x40000000, out=0x60000000, mean=0x70000000)
    a.update(kw)
    assert cal.hcrc_up_kernel(kind, T, a["wu"], a["sc"], a["out"], a["mean"], None) == rc


@pytest.mark.gpu
@pytest.mark.parametrize("T", [1, 2, 5, 8, 12])
def test_up_kernels_alone_reproduce_the_read(cal, T):
    """After a read, either up kernel run alone on the handle's scratch gives the read's out and mean: bitwise
    for the one the read dispatches (the matrix-core kernel, for BF16 weights at every T), within 1e-5 of
    max |out| for the other."""
    import torch

    from bf16_hyper_connection_amd import hcr
    from bf16_hyper_connection_amd import inputs as gen
    from tests.gpu_util import dev, reader_for, to_dev

    print(f"up kernels alone T={T}", flush=True)
    r = reader_for(gen.weight_set(0, 1))
    x = to_dev(gen.activations(1, T))
    ref_o, ref_m = r.read(x)
    torch.cuda.synchronize()
    ref_o, ref_m = ref_o.clone(), ref_m.clone()
    st = torch.cuda.current_stream().cuda_stream
    got = {}
    for kind in (0, 1):
        o = torch.full((T, 4, 2560), float("nan"), device=dev())
        m = torch.full((T, 2560), float("nan"), device=dev())
        rc = cal.hcrc_up_kernel(kind, T, r.w_up.data_ptr(), r.scratch.data_ptr(), o.data_ptr(), m.data_ptr(), st)
        assert rc == HCR_OK, hcr.hcr_strerror(rc)
        torch.cuda.synchronize()
        got[kind] = (o, m)
    dispatched = 1
    assert torch.equal(got[dispatched][0], ref_o) and torch.equal(got[dispatched][1], ref_m)
    scale = float(ref_o.abs().max())
    other = got[1 - dispatched]
    assert float((other[0] - ref_o).abs().max()) <= 1e-5 * scale
    assert float((other[1] - ref_m).abs().max()) <= 1e-5 * scale


@pytest.mark.parametrize("kind,T,kw,rc", [
    (3, 1, {}, HCR_EINVAL),
    (0, 0, {}, HCR_EINVAL),
    (2, 9, {}, HCR_EINVAL),
    (1, 2, dict(x=None), HCR_EINVAL),
    (2, 2, dict(sc=0x40000010), HCR_EALIGN),
    (0, 2, dict(wd=0x10000008), HCR_EALIGN),
])
def test_slab_pair_rejects_before_any_hip_call(cal, kind, T, kw, rc):
    a = dict(FAKE)
    a.update(kw)
    assert cal.hcrc_slab_pair(kind, T, a["wd"], a["wu"], a["wn"], a["sc"], a["x"], None) == rc


@pytest.mark.gpu
@pytest.mark.parametrize("T", [1, 4, 8])
def test_slab_finish_protocol(cal, T):
    """The last-arriver finish of the slab probe: after each call every counter is back to zero, and lo holds
    what the 8th work-group of each row group computed from the 8 slabs' partials (thread t * 10 + r stored
    10 t + r; sums of squares 1): lo[t][r] = 8 (10 t + r mod 10)."""
    import torch

    from bf16_hyper_connection_amd import inputs as gen
    from tests.gpu_util import dev, reader_for, to_dev

    print(f"slab pair T={T}", flush=True)
    r = reader_for(gen.weight_set(0, 2))
    x = to_dev(gen.activations(2, T))
    sc = torch.zeros(256 * 1024, dtype=torch.uint8, device=dev())
    st = torch.cuda.current_stream().cuda_stream
    for rep in range(3):
        for kind in (0, 1, 2):
            rc = cal.hcrc_slab_pair(kind, T, r.w_down.data_ptr(), r.w_up.data_ptr(), r.w_norm.data_ptr(),
                                    sc.data_ptr(), x.data_ptr(), st)
            assert rc == HCR_OK
    torch.cuda.synchronize()
    f = sc.view(torch.float32)
    ss_off, ctr_off = 8 * 16 * 320 * 4, 8 * 16 * 320 * 4 + 8 * 16 * 4 + 256
    lo_off = ctr_off + 256
    assert torch.all(sc.view(torch.int32)[ctr_off // 4: ctr_off // 4 + 32] == 0)
    lo = f[lo_off // 4: lo_off // 4 + T * 320].view(T, 320).cpu()
    t = torch.arange(T).view(T, 1).float()
    rr = (torch.arange(320) % 10).view(1, 320).float()
    assert torch.equal(lo, 8.0 * (10.0 * t + rr))


SLAB_FAKE = dict(FAKE, p=0x60000000, inj=0x68000000, out=0x70000000, mean=0x78000000)


@pytest.mark.parametrize("T,kw,rc", [
    (0, {}, HCR_EINVAL),
    (9, {}, HCR_EINVAL),
    (2, dict(out=None), HCR_EINVAL),
    (2, dict(mean=None), HCR_EINVAL),
    (2, dict(sc=None), HCR_EINVAL),
    (2, dict(wn=None), HCR_EINVAL),
    (2, dict(sc=0x40000080), HCR_EALIGN),
    (2, dict(p=0x60000004), HCR_EALIGN),
    (2, dict(inj=0x68000008), HCR_EALIGN),
    (2, dict(out=0x70000004), HCR_EALIGN),
])
def test_slab_read_rejects_before_any_hip_call(cal, T, kw, rc):
    a = dict(SLAB_FAKE)
    a.update(kw)
    assert cal.hcrc_slab_read(T, a["wd"], a["wu"], a["wn"], a["sc"], a["x"], a["p"], a["inj"], a["out"], a["mean"],
                              None) == rc


@pytest.mark.gpu
@pytest.mark.parametrize("T,pend,inj", [(1, False, False), (2, True, True), (3, False, True), (5, True, False),
                                        (6, True, False), (8, True, True)])
def test_slab_read_matches_the_reference(cal, T, pend, inj):
    """The read in the pages' shape (slab down kernel, last-arriver finish, up kernel on lo): out, mean, lo and
    rs within the read's tolerance of the FP64 reference on every call, the counters back at zero after each,
    and repeated calls (also from a replayed graph) bitwise equal."""
    import numpy as np
    import torch

    import oracle
    from bf16_hyper_connection_amd import hcr
    from bf16_hyper_connection_amd import inputs as gen
    from tests.gpu_util import dev, reader_for, to_dev

    print(f"slab read T={T} pending={pend} inj={inj}", flush=True)
    w = gen.weight_set(0, 3)
    r = reader_for(w)
    x = gen.activations(3, T)
    p = gen.pending(3, T) if pend else None
    ij = gen.injection(3, T) if inj else None
    xd = to_dev(x)
    pd = to_dev(p) if pend else None
    idd = to_dev(ij) if inj else None
    sc = torch.zeros(256 * 1024, dtype=torch.uint8, device=dev())
    out = torch.empty((T, 4, 2560), device=dev())
    mean = torch.empty((T, 2560), device=dev())
    st = torch.cuda.current_stream().cuda_stream

    def call(stream):
        return cal.hcrc_slab_read(T, r.w_down.data_ptr(), r.w_up.data_ptr(), r.w_norm.data_ptr(), sc.data_ptr(),
                                  xd.data_ptr(), pd.data_ptr() if pend else None, idd.data_ptr() if inj else None,
                                  out.data_ptr(), mean.data_ptr(), stream)

    ref = oracle.hc_read(x, w.w_norm, w.w_down, w.w_up, pending=p, inj=ij)
    ctr_off, lo_off, rs_off = 8 * 16 * 320 * 4 + 8 * 16 * 4 + 256, 164864, 185344
    first = None
    for rep in range(3):
        out.fill_(float("nan"))
        mean.fill_(float("nan"))
        rc = call(st)
        assert rc == HCR_OK, hcr.hcr_strerror(rc)
        torch.cuda.synchronize()
        assert torch.all(sc.view(torch.int32)[ctr_off // 4: ctr_off // 4 + 32] == 0), f"counters, call {rep}"
        f = sc.view(torch.float32)
        got = {"out": out.cpu().numpy(), "mean": mean.cpu().numpy(),
               "lo": f[lo_off // 4: lo_off // 4 + T * 320].view(T, 320).cpu().numpy(),
               "rs": f[rs_off // 4: rs_off // 4 + T * 4].view(T, 4).cpu().numpy()}
        for name in ("out", "mean", "lo"):
            err = np.max(np.abs(got[name].astype(np.float64) - ref[name])) / np.max(np.abs(ref[name]))
            assert err <= 1e-4, (name, rep, err)
        assert np.max(np.abs(got["rs"] / ref["rs"] - 1.0)) <= 1e-5
        if first is None:
            first = {k: v.copy() for k, v in got.items()}
        else:
            for k in first:
                assert np.array_equal(first[k], got[k]), (k, rep)
    # captured once, replayed with eager work between: the same bytes
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            assert call(s.cuda_stream) == HCR_OK
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        out.fill_(float("nan"))
        mean.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), first["out"]) and np.array_equal(mean.cpu().numpy(), first["mean"])
        assert torch.all(sc.view(torch.int32)[ctr_off // 4: ctr_off // 4 + 32] == 0)
        r.read(to_dev(gen.activations(4 + rep, T)))
        torch.cuda.synchronize()
