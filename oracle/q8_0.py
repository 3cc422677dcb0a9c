"""FP64 CPU reference of the Q8_0 copies of the read's projections, and of the read on them.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. It shares
no code with the HIP path and imports nothing from it.

What the pages fix, and what this module reads into them
--------------------------------------------------------
Strata PR #2812 (section Summary, and the note on the PR it depends on,
#2810 "STRATA_HC_Q8=1 reads the Q8_0 hyper-connection projections") names a
sibling read that runs the same two-kernel structure on Q8_0 copies of the
two projections, kept in VRAM beside the BF16 weights.  The pages do not
define the Q8_0 block.  The reading taken here is the public GGML Q8_0
format, restated:

* a block is 32 consecutive weights of one row (along the reduction axis K);
* it stores one scale ``d`` as IEEE binary16 and 32 signed 8-bit codes ``q``;
* a weight decodes to ``d * q``;
* quantisation, in binary32 arithmetic: ``amax`` = max |w| over the block,
  ``d = amax / 127``, ``id = 1 / d`` (0 when d = 0), ``q = round(w * id)``
  with ties away from zero, and the stored scale is ``d`` rounded to
  binary16 (nearest, ties to even).  The codes use the binary32 ``d``, not
  the stored binary16 one.

Where floating point decides an integer (the codes), this module takes the
decision in the same binary32 precision as the kernel: numpy ``float32``
arithmetic is IEEE binary32 with round-to-nearest-even.  Everything after
decoding is float64.  Storage here is split: codes int8 [rows][K] and scale
bit patterns uint16 [rows][K/32].
"""

import numpy as np

from .reference import EPS, bf16_bits_to_f64, hc_read_decoded

BLOCK = 32


def fp16_round(v):
    """Round finite float64 values to the nearest IEEE binary16 value (ties to even), as float64.

    binary16: 11 significant bits, exponents -14..15, subnormals down to
    2**-24, largest finite 65504; a value whose rounding exceeds 65504
    overflows to infinity.  Written from the format's definition: with
    |v| = m * 2**(e+1), m in [0.5, 1), the last kept bit is worth 2**(e-10)
    (2**-24 below the normal range); divide by it (exact, a power of two),
    round to the nearest integer with ties to even, multiply back.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)                       # a = m * 2**ex, m in [0.5, 1); e = ex - 1
    e = np.maximum(ex.astype(np.float64) - 1.0, -14.0)
    ulp = np.exp2(e - 10.0)
    r = np.round(a / ulp) * ulp                # np.round: ties to even
    r = np.where(r > 65504.0, np.inf, r)
    return np.copysign(r, v)


def fp16_bits(v):
    """IEEE binary16 bit patterns (uint16) of values that are already binary16 values (float64)."""
    v = np.asarray(v, dtype=np.float64)
    bits = np.zeros(v.shape, dtype=np.uint16)
    sign = np.signbit(v).astype(np.uint16) << np.uint16(15)
    a = np.abs(v)
    inf = np.isinf(a)
    sub = (a < 2.0 ** -14) & ~inf
    norm = ~sub & ~inf
    # subnormal: mantissa = a / 2**-24
    bits[sub] = (a[sub] / 2.0 ** -24).astype(np.uint16)
    if np.any(norm):
        m, ex = np.frexp(a[norm])  # a = m * 2**ex, m in [0.5, 1)
        exp_field = (ex - 1 + 15).astype(np.uint16)
        mant = ((m * 2.0 - 1.0) * 1024.0).astype(np.uint16)
        bits[norm] = (exp_field << np.uint16(10)) | mant
    bits[inf] = np.uint16(0x7C00)
    return bits | sign


def fp16_bits_to_f64(bits):
    """Decode IEEE binary16 bit patterns (uint16) to float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    ex = (b >> 10) & 0x1F
    mant = (b & 0x3FF).astype(np.float64)
    val = np.where(ex == 0, mant * 2.0 ** -24, (1.0 + mant / 1024.0) * np.exp2(ex - 15.0))
    val = np.where(ex == 0x1F, np.where(mant == 0, np.inf, np.nan), val)
    return sign * val


def quantize_q8_0(w_bits):
    """Q8_0 copy of a BF16 matrix: codes int8 [rows][K] and scale bits uint16 [rows][K/32].

    The block rule above, applied to each run of 32 weights along a row.
    w_bits: uint16 BF16 bit patterns [rows][K], K a multiple of 32; weights finite.
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    rows, K = w_bits.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    w = bf16_bits_to_f64(w_bits).astype(np.float32).reshape(rows, K // BLOCK, BLOCK)  # exact
    amax = np.max(np.abs(w), axis=2)                                  # exact
    d = amax / np.float32(127.0)                                       # binary32 division
    with np.errstate(divide="ignore"):
        inv = np.where(d != 0, np.float32(1.0) / np.where(d != 0, d, np.float32(1.0)), np.float32(0.0))
    inv = inv.astype(np.float32)
    v = (w * inv[:, :, None]).astype(np.float32)                       # binary32 product
    v64 = v.astype(np.float64)
    q = np.sign(v64) * np.floor(np.abs(v64) + 0.5)                     # ties away from zero, exact in f64
    codes = q.astype(np.int8).reshape(rows, K)
    scales = fp16_bits(fp16_round(d.astype(np.float64)))
    return codes, scales


def dequantize_q8_0(codes, scale_bits):
    """float64 weights d * q of a Q8_0 copy (codes int8 [rows][K], scale bits uint16 [rows][K/32])."""
    codes = np.asarray(codes, dtype=np.int8)
    rows, K = codes.shape
    d = fp16_bits_to_f64(scale_bits).reshape(rows, K // BLOCK, 1)
    return (d * codes.reshape(rows, K // BLOCK, BLOCK).astype(np.float64)).reshape(rows, K)


def hc_read_q8_0(x, w_norm, down_codes, down_scales, up_codes, up_scales, pending=None, inj=None, eps=EPS):
    """The HC read (norm, down, up, epilogue) on Q8_0 copies of W_down [R][S*d] and W_up [S*d][R].

    The same read as ``reference.hc_read``, with each weight taken as its
    decoded Q8_0 value d * q.  Returns the same dict.
    """
    return hc_read_decoded(x, w_norm, dequantize_q8_0(down_codes, down_scales),
                           dequantize_q8_0(up_codes, up_scales), pending=pending, inj=inj, eps=eps)
