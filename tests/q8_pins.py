"""Pins of the Q8_0 part of the FP64 reference: checks against things other than the reference itself.

The Q8_0 block rule (32 weights of a row, an IEEE binary16 scale d = amax/127
and int8 codes q = round(w / d), ties away from zero, the codes taken with the
binary32 d) is the public GGML format, the reading taken for the pages' Q8_0
copies (Strata PR #2812, Summary and its dependency #2810).  Each ``pin_*``
raises ``AssertionError`` when the functions under test disagree with:

* the IEEE 754 binary16 format: values whose encodings the standard fixes,
  and numpy's own float16 conversion;
* brute force in exact rational arithmetic (``fractions.Fraction``) with
  binary32 and binary16 rounding written out from their definitions;
* blocks whose codes and scales are known by construction (multiples of
  2**-7, rounding ties at a block maximum of 127, an all-zero block);
* the quantisation error bound and the code range;
* the BF16 read on the same weights when the Q8_0 copy is lossless, and the
  closed form with identity-like weights.

``tests/test_oracle_q8.py`` runs them on the reference;
``tests/test_oracle_mutants.py`` runs them on copies with planted mistakes.
"""

from fractions import Fraction

import numpy as np

from bf16_hyper_connection_amd import inputs as gen

# ---------------------------------------------------------------------------
# exact binary32 / binary16 rounding (from the formats' definitions)
# ---------------------------------------------------------------------------


def _round_binary(fr, mant_bits, emin, emax):
    """Round a Fraction to the nearest value with ``mant_bits`` significant bits
    (exponent >= emin, subnormals below; ties to even).  Overflow gives None."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - (mant_bits - 1))
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r >= Fraction(2) ** (emax + 1):
        return None
    return sign * r


def rnd32(fr):
    return _round_binary(fr, 24, -126, 127)


def rnd16(fr):
    return _round_binary(fr, 11, -14, 15)


def brute_force_block(w_exact):
    """(codes, scale) of one block of 32 exact weights, in exact rationals; scale None = overflow."""
    amax = max(abs(v) for v in w_exact)
    d = rnd32(amax / 127)
    inv = rnd32(1 / d) if d != 0 else Fraction(0)
    codes = []
    for v in w_exact:
        p = rnd32(v * inv)
        a = abs(p)
        q = (a + Fraction(1, 2)).numerator // (a + Fraction(1, 2)).denominator
        codes.append(q if p >= 0 else -q)
    return codes, rnd16(d)


def _bf16_exact(bits):
    out = []
    for b in np.asarray(bits, dtype=np.uint16).ravel():
        u = int(b) << 16
        f = np.array([u], dtype=np.uint32).view(np.float32)[0]
        out.append(Fraction(float(f)))
    return out


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

# IEEE 754-2008 binary16 encodings of values the format fixes
FP16_GOLDEN = [
    (1.0, 0x3C00), (-2.0, 0xC000), (65504.0, 0x7BFF), (65519.0, 0x7BFF),  # 65519 rounds down to the max
    (65520.0, 0x7C00),                 # halfway to 2**16: ties to even overflow to +inf
    (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000),  # smallest subnormal; half of it ties to even (0)
    (3.0 * 2.0 ** -26, 0x0001),        # above the half: rounds up to the smallest subnormal
    (2.0 ** -14, 0x0400),              # smallest normal
    (1.0 / 3.0, 0x3555), (2049.0, 0x6800), (2051.0, 0x6802),  # ties to even at spacing 2
    (0.0, 0x0000),
]


def pin_fp16(fp16_round, fp16_bits, fp16_bits_to_f64):
    for v, bits in FP16_GOLDEN:
        r = fp16_round(np.array([v]))
        got = int(fp16_bits(r)[0])
        assert got == bits, (v, hex(got), hex(bits))
        if bits != 0x7C00:
            assert fp16_bits_to_f64(np.array([bits], dtype=np.uint16))[0] == r[0]
    g = np.random.default_rng(11)
    x = (g.standard_normal(200_000) * np.exp2(g.integers(-30, 16, 200_000))).astype(np.float32).astype(np.float64)
    x = x[np.abs(x) < 65504.0]
    lib = x.astype(np.float16)
    r = fp16_round(x)
    assert np.array_equal(r, lib.astype(np.float64)), "binary16 rounding differs from numpy's float16"
    assert np.array_equal(fp16_bits(r), lib.view(np.uint16)), "binary16 encoding differs from numpy's"


def pin_brute_force_blocks(quantize):
    """Every block of the edge matrix and of a normal matrix against exact rational arithmetic."""
    for w in (gen.q8_edge_weights(3, rows=8, K=320), gen.weight_set(3, 0, S=1, d=320, R=4).w_down):
        codes, scales = quantize(w)
        rows, K = w.shape
        for r in range(rows):
            for b in range(K // 32):
                blk = _bf16_exact(w[r, 32 * b:32 * b + 32])
                q_ref, d_ref = brute_force_block(blk)
                assert list(codes[r, 32 * b:32 * b + 32].astype(int)) == q_ref, (r, b)
                bits = int(scales[r, b])
                if d_ref is None:
                    assert bits & 0x7FFF == 0x7C00, (r, b, hex(bits))
                else:
                    got = np.array([bits], dtype=np.uint16).view(np.float16).astype(np.float64)[0]
                    assert Fraction(float(got)) == d_ref, (r, b, float(got), float(d_ref))


def pin_known_blocks(quantize, dequantize):
    """Blocks whose Q8_0 copy is known by construction."""
    g = np.random.default_rng(5)
    # multiples of 2**-7 with a block maximum of 127 * 2**-7: d = 2**-7 exactly, codes = the integers
    k = g.integers(-127, 128, size=(2, 64))
    k[:, 0] = 127
    k[:, 32] = -127
    w = gen.f32_to_bf16_bits((k * 2.0 ** -7).astype(np.float32))
    codes, scales = quantize(w)
    assert np.array_equal(codes.astype(int), k)
    assert np.all(scales == 0x2000)          # binary16 of 2**-7
    assert np.array_equal(dequantize(codes, scales), k * 2.0 ** -7)
    # ties: block maximum 127 gives d = 1 and id = 1, so each +-(n + 1/2) is a tie, taken away from zero
    v = np.array([0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 126.5, -126.5] * 4, dtype=np.float32)
    v[3] = 127.0
    codes, scales = quantize(gen.f32_to_bf16_bits(v[None, :]))
    want = np.array([1, -1, 2, 127, 3, -3, 127, -127] * 4)
    want[11], want[19], want[27] = -2, -2, -2
    assert np.array_equal(codes[0].astype(int), want), codes[0]
    assert scales[0, 0] == 0x3C00            # binary16 of 1
    # all-zero block: scale 0 and codes 0
    codes, scales = quantize(np.zeros((1, 32), dtype=np.uint16))
    assert not np.any(codes) and scales[0, 0] == 0


def pin_error_bound(quantize, dequantize):
    """|w - d16*q| <= d32/2 (1 + 2**-20) + 127 |d32 - d16|, |q| <= 127, and |q| = 127 at the block maximum."""
    w = gen.weight_set(9, 0, S=2, d=640, R=64).w_down
    codes, scales = quantize(w)
    wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    blocks = wf.reshape(-1, 32)
    amax = np.max(np.abs(blocks), axis=1)
    d32 = (amax.astype(np.float32) / np.float32(127.0)).astype(np.float64)
    d16 = scales.reshape(-1).view(np.float16).astype(np.float64)
    err = np.abs(blocks - dequantize(codes, scales).reshape(-1, 32))
    bound = d32 * 0.5 * (1 + 2.0 ** -20) + 127.0 * np.abs(d32 - d16)
    assert np.all(err <= bound[:, None]), float(np.max(err / bound[:, None]))
    c = codes.reshape(-1, 32).astype(int)
    assert np.all(np.abs(c) <= 127)
    at_max = np.abs(c[np.arange(len(c)), np.argmax(np.abs(blocks), axis=1)])
    assert np.all(at_max == 127)


def pin_read_lossless_equals_bf16(read_q8, read_bf16, quantize):
    """On weights the Q8_0 copy holds exactly, the Q8_0 read is the BF16 read."""
    S, d, R, T = 2, 64, 32, 3
    g = np.random.default_rng(21)
    kd = g.integers(-127, 128, size=(R, S * d)); kd[:, ::32] = 127
    ku = g.integers(-127, 128, size=(S * d, R)); ku[:, ::32] = -127
    wd = gen.f32_to_bf16_bits((kd * 2.0 ** -7).astype(np.float32))
    wu = gen.f32_to_bf16_bits((ku * 2.0 ** -9).astype(np.float32))
    wn = gen.weight_set(21, 0, S=S, d=d, R=R).w_norm
    x, p, inj = gen.activations(21, T, S=S, d=d), gen.pending(21, T, S=S, d=d), gen.injection(21, T, R=R)
    cd, sd = quantize(wd)
    cu, su = quantize(wu)
    a = read_q8(x, wn, cd, sd, cu, su, pending=p, inj=inj)
    b = read_bf16(x, wn, wd, wu, pending=p, inj=inj)
    for key in ("out", "mean", "lo", "rs"):
        assert np.array_equal(a[key], b[key]), key


def pin_read_closed_form(read_q8, quantize):
    """Identity-like weights of value 127/128 (held exactly): lo[r] = (127/128) sum_s rs_s x_s[r] w_norm_s[r],
    u_s[c] = (127/128) lo[c mod R], out_s = sigmoid(lo[s]) u_s, mean = average over s."""
    S, d, R, T = 2, 64, 32, 2
    c = 127.0 / 128.0
    wd = np.zeros((R, S * d), dtype=np.float32)
    for s in range(S):
        wd[np.arange(R), s * d + np.arange(R)] = c
    wu = np.zeros((S * d, R), dtype=np.float32)
    wu[np.arange(S * d), np.arange(S * d) % d % R] = c
    wn = gen.weight_set(31, 0, S=S, d=d, R=R).w_norm.astype(np.float64)
    x = gen.activations(31, T, S=S, d=d).astype(np.float64)
    cd, sd = quantize(gen.f32_to_bf16_bits(wd))
    cu, su = quantize(gen.f32_to_bf16_bits(wu))
    got = read_q8(x, wn, cd, sd, cu, su)
    rs = 1.0 / np.sqrt(np.mean(x * x, axis=2) + 1e-6)
    lo = c * np.einsum("ts,tsr,sr->tr", rs, x[:, :, :R], wn[:, :R])
    u = c * lo[:, np.arange(d) % R]
    gate = 1.0 / (1.0 + np.exp(-lo[:, :S]))
    out = gate[:, :, None] * u[:, None, :]
    assert np.allclose(got["lo"], lo, rtol=1e-13, atol=0)
    assert np.allclose(got["out"], out, rtol=1e-12, atol=1e-300)
    assert np.allclose(got["mean"], out.mean(axis=1), rtol=1e-12, atol=1e-300)


def all_pins(fp16_round, fp16_bits, fp16_bits_to_f64, quantize, dequantize, read_q8, read_bf16):
    """(name, thunk) pairs running every pin on the given functions."""
    return [
        ("fp16", lambda: pin_fp16(fp16_round, fp16_bits, fp16_bits_to_f64)),
        ("brute_force_blocks", lambda: pin_brute_force_blocks(quantize)),
        ("known_blocks", lambda: pin_known_blocks(quantize, dequantize)),
        ("error_bound", lambda: pin_error_bound(quantize, dequantize)),
        ("read_lossless_equals_bf16", lambda: pin_read_lossless_equals_bf16(read_q8, read_bf16, quantize)),
        ("read_closed_form", lambda: pin_read_closed_form(read_q8, quantize)),
    ]
