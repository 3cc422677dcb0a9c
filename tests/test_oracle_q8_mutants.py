"""Planted mistakes in copies of the Q8_0 reference must each fail at least one Q8_0 pin.

Each mutant is the reference quantiser or decoder with one plausible slip in
the block rule; the mistake is planted in a CPU copy, never in the HIP path.
"""

import numpy as np
import pytest

import oracle
from oracle import q8_0
from tests import q8_pins


def _quantize(ties="away", divisor=127.0, codes_from="f32", scale_round="nearest", amax="abs", span=32):
    """A copy of the reference quantiser with one step replaced."""
    def quantize(w_bits):
        w_bits = np.asarray(w_bits, dtype=np.uint16)
        rows, K = w_bits.shape
        w = q8_0.bf16_bits_to_f64(w_bits).astype(np.float32).reshape(rows, K // 32, 32)
        part = w[:, :, :span]
        m = np.max(np.abs(part), axis=2) if amax == "abs" else np.max(part, axis=2)
        d = (m / np.float32(divisor)).astype(np.float32)
        if scale_round == "nearest":
            d16 = q8_0.fp16_round(d.astype(np.float64))
        else:  # toward zero: drop the bits below the 11th
            d16 = np.asarray(d, dtype=np.float64)
            _, ex = np.frexp(d16)
            ulp = np.exp2(np.maximum(ex - 1.0, -14.0) - 10.0)
            d16 = np.trunc(d16 / ulp) * ulp
        dq = d if codes_from == "f32" else d16.astype(np.float32)
        with np.errstate(divide="ignore"):
            inv = np.where(dq != 0, np.float32(1.0) / np.where(dq != 0, dq, np.float32(1.0)), np.float32(0.0))
        v = (w * inv.astype(np.float32)[:, :, None]).astype(np.float32).astype(np.float64)
        q = np.sign(v) * np.floor(np.abs(v) + 0.5) if ties == "away" else np.round(v)
        q = np.clip(q, -128, 127)
        return q.astype(np.int8).reshape(rows, K), q8_0.fp16_bits(d16)
    return quantize


def _dequantize_blocks_down_columns(codes, scale_bits):
    codes = np.asarray(codes, dtype=np.int8)
    rows, K = codes.shape
    d = q8_0.fp16_bits_to_f64(scale_bits).reshape(-1)          # scales taken in column-major block order
    d = d.reshape(K // 32, rows).T.reshape(rows, K // 32, 1)
    return (d * codes.reshape(rows, K // 32, 32).astype(np.float64)).reshape(rows, K)


MUTANTS = {
    "ties_to_even": dict(quantize=_quantize(ties="even")),
    "divisor_128": dict(quantize=_quantize(divisor=128.0)),
    "codes_from_binary16_scale": dict(quantize=_quantize(codes_from="f16")),
    "scale_truncated": dict(quantize=_quantize(scale_round="zero")),
    "signed_maximum": dict(quantize=_quantize(amax="signed")),
    "maximum_over_half_block": dict(quantize=_quantize(span=16)),
    "scales_in_wrong_block_order": dict(dequantize=_dequantize_blocks_down_columns),
}


def _pins(quantize=q8_0.quantize_q8_0, dequantize=q8_0.dequantize_q8_0):
    def read_q8(x, w_norm, cd, sd, cu, su, pending=None, inj=None):
        return oracle.hc_read_decoded(x, w_norm, dequantize(cd, sd), dequantize(cu, su), pending=pending, inj=inj)
    return q8_pins.all_pins(q8_0.fp16_round, q8_0.fp16_bits, q8_0.fp16_bits_to_f64, quantize, dequantize,
                            read_q8, oracle.hc_read)


def test_unmutated_copy_passes_every_pin():
    for _, pin in _pins(quantize=_quantize()):
        pin()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_q8_mutant_fails_a_pin(name):
    failed = []
    for pname, pin in _pins(**MUTANTS[name]):
        try:
            pin()
        except (AssertionError, ValueError) as e:  # noqa: PERF203
            failed.append((pname, str(e)[:80]))
    assert failed, f"mutant {name} passed every pin"
