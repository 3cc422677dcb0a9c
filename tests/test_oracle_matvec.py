"""The skinny BF16 matvec reference against its pins, and planted mistakes against the pins (CPU only)."""

import numpy as np
import pytest

import oracle
from tests import matvec_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=[p.__name__ for p in pins.ALL_PINS])
def test_matvec_reference_pin(pin):
    pin(oracle.matvec_bf16)


def _w(bits):
    return oracle.bf16_bits_to_f64(bits)


MUTANTS = {
    "transposed_weights": lambda w, x: np.asarray(x, np.float64) @ _w(w)[:, :].T[:, ::-1],
    "reversed_k": lambda w, x: np.asarray(x, np.float64)[:, ::-1] @ _w(w).T,
    "weights_rounded_to_fp16": lambda w, x: np.asarray(x, np.float64) @ _w(w).astype(np.float16).astype(np.float64).T,
    "last_column_dropped": lambda w, x: np.asarray(x, np.float64)[:, :-1] @ _w(w)[:, :-1].T,
    "x_rounded_to_bf16": lambda w, x: (np.asarray(x, np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
    .astype(np.float64) @ _w(w).T,
    "columns_summed": lambda w, x: np.repeat(np.sum(np.asarray(x, np.float64), axis=0, keepdims=True),
                                             np.asarray(x).shape[0], axis=0) @ _w(w).T,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_matvec_mutant_fails_a_pin(name):
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(MUTANTS[name])
        except (AssertionError, ValueError):  # noqa: PERF203
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
