"""ctypes binding of libhcr.so, the BF16 hyper-connection read and its Q8_0 sibling (C ABI in include/hcr.h).

Argument marshalling only: tensors are passed as raw device pointers and
torch's current HIP stream; every step of the read runs in the library's
kernels.  There is no fallback: if the library is missing or a call fails,
an exception is raised.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# HCR_LIB names another build of the same C ABI (the tests run the host-sanitizer build through it)
LIB_PATH = os.environ.get("HCR_LIB") or os.path.join(_PKG, "libhcr.so")

HCR_OK, HCR_EINVAL, HCR_EALIGN, HCR_ESCRATCH, HCR_EALIAS, HCR_EHIP = 0, -1, -2, -3, -4, -5

_lib = None


class HCRError(RuntimeError):
    def __init__(self, rc, what):
        super().__init__(f"{what}: {hcr_strerror(rc)} (code {rc})")
        self.rc = rc


def lib():
    """The loaded libhcr.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, ip = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.hcr_scratch_bytes.restype = sz
        L.hcr_scratch_bytes.argtypes = []
        L.hcr_scratch_layout.restype = ip
        L.hcr_scratch_layout.argtypes = [ctypes.POINTER(sz), ctypes.POINTER(sz)]
        L.hcr_geometry.restype = ip
        L.hcr_geometry.argtypes = [ctypes.POINTER(ip)] * 4
        L.hcr_create.restype = ip
        L.hcr_create.argtypes = [vp, vp, vp, vp, sz, ctypes.POINTER(vp)]
        L.hcr_create_q8_0.restype = ip
        L.hcr_create_q8_0.argtypes = [vp, vp, vp, vp, vp, vp, sz, ctypes.POINTER(vp)]
        L.hcr_quantize_q8_0.restype = ip
        L.hcr_quantize_q8_0.argtypes = [vp, ip, ip, vp, vp, vp]
        L.hcr_matvec_bf16.restype = ip
        L.hcr_matvec_bf16.argtypes = [vp, ip, ip, ip, vp, vp, vp]
        L.hcr_read.restype = ip
        L.hcr_read.argtypes = [vp, ip, vp, vp, vp, vp, vp, vp]
        L.hcr_read_static.restype = ip
        L.hcr_read_static.argtypes = [vp, vp, vp, ip, vp, vp, vp, vp, vp, vp]
        L.hcr_destroy.restype = None
        L.hcr_destroy.argtypes = [vp]
        L.hcr_strerror.restype = ctypes.c_char_p
        L.hcr_strerror.argtypes = [ip]
        _lib = L
    return _lib


# ---- the C entry points, same names ----

def hcr_scratch_bytes():
    return int(lib().hcr_scratch_bytes())


def hcr_scratch_layout():
    lo, rs = ctypes.c_size_t(), ctypes.c_size_t()
    rc = lib().hcr_scratch_layout(ctypes.byref(lo), ctypes.byref(rs))
    if rc != HCR_OK:
        raise HCRError(rc, "hcr_scratch_layout")
    return lo.value, rs.value


def hcr_geometry():
    v = [ctypes.c_int() for _ in range(4)]
    lib().hcr_geometry(*[ctypes.byref(x) for x in v])
    return tuple(x.value for x in v)


def hcr_strerror(rc):
    return lib().hcr_strerror(int(rc)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _raw(p):
    return None if p is None else ctypes.c_void_p(int(p))


def hcr_create(w_down, w_up, w_norm, scratch, scratch_bytes):
    """Raw-pointer form (ints or None); returns the handle as an int."""
    h = ctypes.c_void_p()
    rc = lib().hcr_create(_raw(w_down), _raw(w_up), _raw(w_norm), _raw(scratch), scratch_bytes, ctypes.byref(h))
    if rc != HCR_OK:
        raise HCRError(rc, "hcr_create")
    return h.value


def hcr_create_q8_0(down_codes, down_scales, up_codes, up_scales, w_norm, scratch, scratch_bytes):
    """Raw-pointer form (ints or None); returns the handle as an int."""
    h = ctypes.c_void_p()
    rc = lib().hcr_create_q8_0(_raw(down_codes), _raw(down_scales), _raw(up_codes), _raw(up_scales), _raw(w_norm),
                               _raw(scratch), scratch_bytes, ctypes.byref(h))
    if rc != HCR_OK:
        raise HCRError(rc, "hcr_create_q8_0")
    return h.value


def hcr_quantize_q8_0(w, rows, cols, codes, scales, stream):
    """Raw-pointer form (ints or None); returns the status code without raising."""
    return lib().hcr_quantize_q8_0(_raw(w), int(rows), int(cols), _raw(codes), _raw(scales), _raw(stream))


def quantize_q8_0(w, stream=None):
    """Q8_0 copy of a contiguous BF16 device matrix [rows][cols]: (codes int8 [rows][cols],
    scales int16 [rows][cols/32] holding binary16 bit patterns), made on the device."""
    if w.dim() != 2 or not w.is_contiguous() or not w.is_cuda or w.element_size() != 2:
        raise ValueError("w: a contiguous 2-D BF16 (2-byte) device tensor")
    rows, cols = w.shape
    if cols % 32:
        raise ValueError("cols must be a multiple of 32")
    codes = torch.empty((rows, cols), dtype=torch.int8, device=w.device)
    scales = torch.empty((rows, cols // 32), dtype=torch.int16, device=w.device)
    st = current_stream_ptr(w.device) if stream is None else stream
    rc = hcr_quantize_q8_0(w.data_ptr(), rows, cols, codes.data_ptr(), scales.data_ptr(), st)
    if rc != HCR_OK:
        raise HCRError(rc, "hcr_quantize_q8_0")
    return codes, scales


def hcr_matvec_bf16(w, rows, cols, T, x, y, stream):
    """Raw-pointer form of hcr_matvec_bf16 (ints or None); returns the status code without raising."""
    return lib().hcr_matvec_bf16(_raw(w), int(rows), int(cols), int(T), _raw(x), _raw(y), _raw(stream))


def matvec_bf16(w, x, y=None, stream=None):
    """y [T][rows] = x [T][cols] times W^T, W a contiguous BF16 (2-byte) device matrix [rows][cols]."""
    if w.dim() != 2 or not w.is_contiguous() or not w.is_cuda or w.element_size() != 2:
        raise ValueError("w: a contiguous 2-D BF16 (2-byte) device tensor")
    rows, cols = w.shape
    if x.dim() != 2 or x.shape[1] != cols or x.dtype != torch.float32 or not x.is_contiguous() or x.device != w.device:
        raise ValueError(f"x: contiguous float32 [T][{cols}] on {w.device}")
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, rows), dtype=torch.float32, device=w.device)
    if tuple(y.shape) != (T, rows) or y.dtype != torch.float32 or not y.is_contiguous() or y.device != w.device:
        raise ValueError(f"y: contiguous float32 [{T}][{rows}] on {w.device}")
    st = current_stream_ptr(w.device) if stream is None else stream
    rc = hcr_matvec_bf16(w.data_ptr(), rows, cols, T, x.data_ptr(), y.data_ptr(), st)
    if rc != HCR_OK:
        raise HCRError(rc, "hcr_matvec_bf16")
    return y


def hcr_read(h, T, x, pending, inj, out, mean, stream):
    """Raw-pointer form (ints or None); returns the status code without raising."""
    return lib().hcr_read(_raw(h), int(T), _raw(x), _raw(pending), _raw(inj), _raw(out), _raw(mean), _raw(stream))


def hcr_read_static(w_down, w_up, w_norm, T, x, pending, inj, out, mean, stream):
    """Raw-pointer form (ints or None) of the read on the library's own scratch; returns the status code
    without raising."""
    return lib().hcr_read_static(_raw(w_down), _raw(w_up), _raw(w_norm), int(T), _raw(x), _raw(pending), _raw(inj),
                                 _raw(out), _raw(mean), _raw(stream))


def hcr_destroy(h):
    lib().hcr_destroy(_raw(h))


def current_stream_ptr(device=None):
    return torch.cuda.current_stream(device).cuda_stream


class HCRead:
    """One weight set (one layer half) and its scratch, bound to a handle.

    w_down: [320][10240] and w_up: [10240][320] BF16 (torch.bfloat16, or the raw
    bit patterns as int16/uint16), w_norm: [4][2560] float32, all on one device.
    """

    def __init__(self, w_down, w_up, w_norm):
        self._init_common(w_down, w_up, w_norm)
        self.handle = hcr_create(w_down.data_ptr(), w_up.data_ptr(), w_norm.data_ptr(),
                                 self.scratch.data_ptr(), self.scratch.numel())

    def _init_common(self, w_down, w_up, w_norm, q8=False):
        S, d, R, self.t_max = hcr_geometry()
        for name, t, shape in (("w_down", w_down, (R, S * d)), ("w_up", w_up, (S * d, R)),
                               ("w_norm", w_norm, (S, d))):
            if tuple(t.shape) != shape or not t.is_contiguous() or not t.is_cuda:
                raise ValueError(f"{name}: expected a contiguous device tensor of shape {shape}")
        esize = 1 if q8 else 2
        if w_down.element_size() != esize or w_up.element_size() != esize or w_norm.dtype != torch.float32:
            raise ValueError("weights: BF16 (2-byte) projections or int8 Q8_0 codes, and a float32 w_norm")
        self.geometry = (S, d, R)
        self.device = w_down.device
        self.w_down, self.w_up, self.w_norm = w_down, w_up, w_norm
        self.scratch = torch.empty(hcr_scratch_bytes(), dtype=torch.uint8, device=self.device)
        self._destroy_fn, self._vp = lib().hcr_destroy, ctypes.c_void_p

    @classmethod
    def q8_0(cls, down_codes, down_scales, up_codes, up_scales, w_norm):
        """A reader of Q8_0 copies (as ``quantize_q8_0`` makes them) instead of BF16 weights."""
        self = cls.__new__(cls)
        self._init_common(down_codes, up_codes, w_norm, q8=True)
        S, d, R = self.geometry
        for name, t, shape in (("down_scales", down_scales, (R, S * d // 32)), ("up_scales", up_scales, (S * d, R // 32))):
            if tuple(t.shape) != shape or not t.is_contiguous() or t.element_size() != 2 or t.device != self.device:
                raise ValueError(f"{name}: expected contiguous 2-byte {shape} on {self.device}")
        self.scales = (down_scales, up_scales)
        self.handle = hcr_create_q8_0(down_codes.data_ptr(), down_scales.data_ptr(), up_codes.data_ptr(),
                                      up_scales.data_ptr(), w_norm.data_ptr(), self.scratch.data_ptr(),
                                      self.scratch.numel())
        return self

    def __del__(self):
        # references bound at creation: at interpreter exit this module's globals may already be gone
        h, fn, vp = getattr(self, "handle", None), getattr(self, "_destroy_fn", None), getattr(self, "_vp", None)
        if h and fn is not None and vp is not None:
            fn(vp(h))
            self.handle = None

    def read(self, x, pending=None, inj=None, out=None, mean=None, stream=None):
        """Enqueue one read of T = x.shape[0] tokens on torch's current stream (or on ``stream``, a raw
        hipStream_t); returns (out, mean).  out and mean allocated here belong to torch's current stream:
        with another ``stream``, pass them in (or record them on that stream) so that torch does not reuse
        their memory before the read has run."""
        S, d, R = self.geometry
        T = x.shape[0]
        if out is None:
            out = torch.empty((T, S, d), dtype=torch.float32, device=self.device)
        if mean is None:
            mean = torch.empty((T, d), dtype=torch.float32, device=self.device)
        for name, t, shape in (("x", x, (T, S, d)), ("pending", pending, (T, S, d)), ("inj", inj, (T, R)),
                               ("out", out, (T, S, d)), ("mean", mean, (T, d))):
            if t is None:
                continue
            if tuple(t.shape) != shape or t.dtype != torch.float32 or not t.is_contiguous() or t.device != self.device:
                raise ValueError(f"{name}: expected contiguous float32 {shape} on {self.device}")
        st = current_stream_ptr(self.device) if stream is None else stream
        rc = lib().hcr_read(ctypes.c_void_p(self.handle), int(T), _ptr(x), _ptr(pending), _ptr(inj),
                            _ptr(out), _ptr(mean), ctypes.c_void_p(st))
        if rc != HCR_OK:
            raise HCRError(rc, "hcr_read")
        return out, mean

    def last_lo_rs(self, T):
        """lo [T][320] and rs [T][4] of the last read, read back from the scratch (after it completes)."""
        S, d, R = self.geometry
        lo_off, rs_off = hcr_scratch_layout()
        f = self.scratch.view(torch.float32)
        lo = f[lo_off // 4: lo_off // 4 + T * R].view(T, R)
        rs = f[rs_off // 4: rs_off // 4 + T * S].view(T, S)
        return lo, rs
