"""The C ABI on the host: the library loads, exports what include/hcr.h declares, and
rejects bad arguments before any HIP call (no GPU is used by these tests)."""

import ctypes

import pytest

from bf16_hyper_connection_amd import hcr
from tests.libhcr_util import declared_functions, ensure_built


@pytest.fixture(scope="module")
def lib():
    return ensure_built()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"hcr_create", "hcr_read", "hcr_destroy", "hcr_scratch_bytes", "hcr_strerror"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"libhcr.so does not export {n}"


def test_geometry_and_scratch(lib):
    assert hcr.hcr_geometry() == (4, 2560, 320, 16)
    n = hcr.hcr_scratch_bytes()
    lo, rs = hcr.hcr_scratch_layout()
    assert n % 256 == 0 and lo % 256 == 0 and rs % 256 == 0
    assert lo + 16 * 320 * 4 <= rs and rs + 16 * 4 * 4 <= n


def test_strerror(lib):
    for rc in (0, -1, -2, -3, -4, -5):
        assert hcr.hcr_strerror(rc) and hcr.hcr_strerror(rc) != hcr.hcr_strerror(-99)


# Fake, never-dereferenced device addresses: the checks below fail before any HIP call.
MB = 1 << 20
WD, WU, WN, SC = 0x10000000, 0x20000000, 0x30000000, 0x40000000
X, P, I, O, M = 0x50000000, 0x60000000, 0x70000000, 0x80000000, 0x90000000


def _create(**kw):
    a = dict(w_down=WD, w_up=WU, w_norm=WN, scratch=SC, scratch_bytes=hcr.hcr_scratch_bytes())
    a.update(kw)
    return hcr.hcr_create(a["w_down"], a["w_up"], a["w_norm"], a["scratch"], a["scratch_bytes"])


@pytest.mark.parametrize("kw,rc", [
    (dict(w_down=None), hcr.HCR_EINVAL),
    (dict(w_up=None), hcr.HCR_EINVAL),
    (dict(w_norm=None), hcr.HCR_EINVAL),
    (dict(scratch=None), hcr.HCR_EINVAL),
    (dict(w_down=WD + 8), hcr.HCR_EALIGN),
    (dict(w_norm=WN + 4), hcr.HCR_EALIGN),
    (dict(scratch=SC + 16), hcr.HCR_EALIGN),
    (dict(scratch_bytes=1024), hcr.HCR_ESCRATCH),
    (dict(scratch=WD + MB), hcr.HCR_EALIAS),       # inside w_down
])
def test_create_rejects(lib, kw, rc):
    with pytest.raises(hcr.HCRError) as e:
        _create(**kw)
    assert e.value.rc == rc


def test_create_null_out(lib):
    assert lib.hcr_create(ctypes.c_void_p(WD), ctypes.c_void_p(WU), ctypes.c_void_p(WN), ctypes.c_void_p(SC),
                          hcr.hcr_scratch_bytes(), None) == hcr.HCR_EINVAL


T_BYTES = 4 * 2560 * 4


@pytest.mark.parametrize("T,args,rc", [
    (17, {}, hcr.HCR_EINVAL),
    (-1, {}, hcr.HCR_EINVAL),
    (2, dict(x=None), hcr.HCR_EINVAL),
    (2, dict(out=None), hcr.HCR_EINVAL),
    (2, dict(mean=None), hcr.HCR_EINVAL),
    (2, dict(x=X + 4), hcr.HCR_EALIGN),
    (2, dict(pending=P + 8), hcr.HCR_EALIGN),
    (2, dict(inj=I + 12), hcr.HCR_EALIGN),
    (2, dict(mean=M + 4), hcr.HCR_EALIGN),
    (2, dict(out=X + 16), hcr.HCR_EALIAS),             # partial overlap with x
    (2, dict(out=P + T_BYTES), hcr.HCR_EALIAS),        # partial overlap with pending (T = 2)
    (2, dict(mean=O + 64), hcr.HCR_EALIAS),            # mean inside out
    (2, dict(mean=X), hcr.HCR_EALIAS),                 # mean on x
    (2, dict(out=SC), hcr.HCR_EALIAS),                 # out on the scratch
    (2, dict(out=WU), hcr.HCR_EALIAS),                 # out on the weights
    (2, dict(inj=SC + 256), hcr.HCR_EALIAS),           # inj on the scratch
    (2, dict(mean=I), hcr.HCR_EALIAS),                 # mean on inj
])
def test_read_rejects_before_any_hip_call(lib, T, args, rc):
    h = _create()
    try:
        a = dict(x=X, pending=P, inj=I, out=O, mean=M)
        a.update(args)
        got = hcr.hcr_read(h, T, a["x"], a["pending"], a["inj"], a["out"], a["mean"], None)
        assert got == rc, (got, hcr.hcr_strerror(got))
    finally:
        hcr.hcr_destroy(h)


def test_read_null_handle_and_empty(lib):
    assert hcr.hcr_read(None, 1, X, None, None, O, M, None) == hcr.HCR_EINVAL
    h = _create()
    try:
        # T = 0: an empty read enqueues nothing, even with null buffers
        assert hcr.hcr_read(h, 0, None, None, None, None, None, None) == hcr.HCR_OK
    finally:
        hcr.hcr_destroy(h)


def test_destroy_null_is_noop(lib):
    hcr.hcr_destroy(None)


# ---- Q8_0 entry points (rejections only: a valid call would launch a kernel)
QD, QDS, QU, QUS = 0xA0000000, 0xB0000000, 0xC0000000, 0xD0000000


def _create_q8(**kw):
    a = dict(dc=QD, ds=QDS, uc=QU, us=QUS, w_norm=WN, scratch=SC, scratch_bytes=hcr.hcr_scratch_bytes())
    a.update(kw)
    return hcr.hcr_create_q8_0(a["dc"], a["ds"], a["uc"], a["us"], a["w_norm"], a["scratch"], a["scratch_bytes"])


@pytest.mark.parametrize("kw,rc", [
    (dict(dc=None), hcr.HCR_EINVAL),
    (dict(ds=None), hcr.HCR_EINVAL),
    (dict(us=None), hcr.HCR_EINVAL),
    (dict(ds=QDS + 2), hcr.HCR_EALIGN),
    (dict(uc=QU + 8), hcr.HCR_EALIGN),
    (dict(scratch_bytes=256), hcr.HCR_ESCRATCH),
    (dict(scratch=QUS + 4096), hcr.HCR_EALIAS),   # inside the up scales (10240 x 10 x 2 bytes)
    (dict(scratch=QD + MB), hcr.HCR_EALIAS),      # inside the down codes
])
def test_create_q8_0_rejects(lib, kw, rc):
    with pytest.raises(hcr.HCRError) as e:
        _create_q8(**kw)
    assert e.value.rc == rc


def test_q8_0_read_rejects_out_on_scales(lib):
    h = _create_q8()
    try:
        assert hcr.hcr_read(h, 1, X, None, None, QDS, M, None) == hcr.HCR_EALIAS
        assert hcr.hcr_read(h, 1, X, None, None, O, QUS + 64, None) == hcr.HCR_EALIAS
        assert hcr.hcr_read(h, 17, X, None, None, O, M, None) == hcr.HCR_EINVAL
    finally:
        hcr.hcr_destroy(h)


@pytest.mark.parametrize("args,rc", [
    (dict(w=None), hcr.HCR_EINVAL),
    (dict(rows=0), hcr.HCR_EINVAL),
    (dict(cols=48), hcr.HCR_EINVAL),          # not a multiple of 32
    (dict(cols=-32), hcr.HCR_EINVAL),
    (dict(codes=None), hcr.HCR_EINVAL),
    (dict(w=WD + 8), hcr.HCR_EALIGN),
    (dict(scales=QDS + 2), hcr.HCR_EALIGN),
    (dict(codes=WD + 4096), hcr.HCR_EALIAS),  # codes inside w
    (dict(scales=QD + 1024), hcr.HCR_EALIAS), # scales inside codes
])
def test_quantize_q8_0_rejects_before_any_hip_call(lib, args, rc):
    a = dict(w=WD, rows=320, cols=10240, codes=QD, scales=QDS)
    a.update(args)
    assert hcr.hcr_quantize_q8_0(a["w"], a["rows"], a["cols"], a["codes"], a["scales"], None) == rc


@pytest.mark.parametrize("args,rc", [
    (dict(w=None), hcr.HCR_EINVAL),
    (dict(x=None), hcr.HCR_EINVAL),
    (dict(y=None), hcr.HCR_EINVAL),
    (dict(rows=0), hcr.HCR_EINVAL),
    (dict(cols=2564), hcr.HCR_EINVAL),          # not a multiple of 8
    (dict(cols=3080), hcr.HCR_EINVAL),          # more than 3072
    (dict(T=5), hcr.HCR_EINVAL),
    (dict(T=-1), hcr.HCR_EINVAL),
    (dict(w=WD + 8), hcr.HCR_EALIGN),
    (dict(x=X + 4), hcr.HCR_EALIGN),
    (dict(y=O + 4), hcr.HCR_EALIGN),
    (dict(y=WD + 4096), hcr.HCR_EALIAS),        # y inside w
    (dict(y=X + 16), hcr.HCR_EALIAS),           # y overlapping x
])
def test_matvec_rejects_before_any_hip_call(lib, args, rc):
    a = dict(w=WD, rows=12288, cols=2560, T=2, x=X, y=O)
    a.update(args)
    assert hcr.hcr_matvec_bf16(a["w"], a["rows"], a["cols"], a["T"], a["x"], a["y"], None) == rc


def test_matvec_empty_is_noop(lib):
    assert hcr.hcr_matvec_bf16(None, 0, 0, 0, None, None, None) == hcr.HCR_OK


def test_source_hash_ignores_comments_only():
    from bf16_hyper_connection_amd import build
    a = build._code_only('int a = 1;  // note\n/* block\n comment */ int b = 2;')
    b = build._code_only('int a = 1;\nint b = 2;  /* other */')
    assert a == b
    assert build._code_only('const char* s = "// not a comment";') == 'const char* s = "// not a comment";'
    assert build._code_only("int a = 1;") != build._code_only("int a = 2;")


# ---- the read on the library's own scratch (rejections only: a valid call would launch kernels)
@pytest.mark.parametrize("T,kw,rc", [
    (17, {}, hcr.HCR_EINVAL),
    (-1, {}, hcr.HCR_EINVAL),
    (2, dict(w_down=None), hcr.HCR_EINVAL),
    (2, dict(w_norm=None), hcr.HCR_EINVAL),
    (2, dict(x=None), hcr.HCR_EINVAL),
    (2, dict(mean=None), hcr.HCR_EINVAL),
    (2, dict(w_up=WU + 8), hcr.HCR_EALIGN),
    (2, dict(x=X + 4), hcr.HCR_EALIGN),
    (2, dict(out=X + 16), hcr.HCR_EALIAS),      # partial overlap with x
    (2, dict(mean=O + 64), hcr.HCR_EALIAS),     # mean inside out
    (2, dict(out=WD + MB), hcr.HCR_EALIAS),     # out on the weights
    (2, dict(mean=WN), hcr.HCR_EALIAS),         # mean on w_norm
])
def test_read_static_rejects_before_any_hip_call(lib, T, kw, rc):
    a = dict(w_down=WD, w_up=WU, w_norm=WN, x=X, pending=P, inj=I, out=O, mean=M)
    a.update(kw)
    got = hcr.hcr_read_static(a["w_down"], a["w_up"], a["w_norm"], T, a["x"], a["pending"], a["inj"], a["out"],
                              a["mean"], None)
    assert got == rc, (got, hcr.hcr_strerror(got))


def test_read_static_empty_is_noop(lib):
    assert hcr.hcr_read_static(None, None, None, 0, None, None, None, None, None, None) == hcr.HCR_OK
