"""The Q8_0 part of the FP64 reference against its pins (CPU only)."""

import pytest

import oracle
from oracle import q8_0
from tests import q8_pins

PINS = q8_pins.all_pins(q8_0.fp16_round, q8_0.fp16_bits, q8_0.fp16_bits_to_f64, q8_0.quantize_q8_0,
                        q8_0.dequantize_q8_0, q8_0.hc_read_q8_0, oracle.hc_read)


@pytest.mark.parametrize("name,pin", PINS, ids=[n for n, _ in PINS])
def test_q8_reference_pin(name, pin):
    pin()
