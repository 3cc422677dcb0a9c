"""The FP64 reference against its pins (CPU only)."""

import json
import os

import numpy as np
import pytest

import oracle
from bf16_hyper_connection_amd import inputs as gen
from tests import oracle_pins as pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.hc_read)


def test_bf16_decode_known_patterns():
    """Bit patterns whose values follow from the binary32 layout by hand."""
    with open(os.path.join(GOLDEN, "bf16_patterns.json")) as fh:
        cases = json.load(fh)["cases"]
    bits = np.array([int(c["bits"], 16) for c in cases], dtype=np.uint16)
    vals = oracle.bf16_bits_to_f64(bits)
    for c, v in zip(cases, vals):
        want = float.fromhex(c["value_hex"])
        assert v == want, (c, v)


def test_closed_form_real_geometry():
    """The identity-like closed form at the pages' geometry (4 x 2560 streams, R = 320)."""
    (x, wn, wd, wu, p, inj), ref = pins.closed_form_case(gen.S_STREAMS, gen.D_STREAM, gen.R_DOWN, 2)
    got = oracle.hc_read(x, wn, wd, wu, pending=p, inj=inj)
    for key in ("rs", "lo", "out", "mean"):
        scale = np.max(np.abs(ref[key]))
        assert np.max(np.abs(got[key] - ref[key])) <= 1e-12 * scale, key


def test_geometry_matches_pages():
    """The generator's geometry against the figures the pages print (tests/golden/geometry.json)."""
    with open(os.path.join(GOLDEN, "geometry.json")) as fh:
        g = json.load(fh)
    assert gen.S_STREAMS == g["streams"]
    assert gen.D_STREAM == 2 * g["slab_columns_half_stream"]
    assert gen.R_DOWN == g["up_K"]
    assert gen.S_STREAMS * 16 == g["up_rows_per_16_columns"]
    assert gen.D_STREAM == g["engine_inputs"]
    w_bytes = 2 * (gen.R_DOWN * gen.S_STREAMS * gen.D_STREAM) * 2
    assert abs(w_bytes / 1e6 - g["weights_MB_per_read"]) < 0.5
    assert gen.T_MAX == max(g["tokens_tested"])


def test_real_geometry_shapes_and_finite():
    c = gen.single_read(0)
    w = c["weights"][0]
    r = oracle.hc_read(c["x"], w.w_norm, w.w_down, w.w_up)
    assert r["out"].shape == (1, 4, 2560) and r["mean"].shape == (1, 2560)
    assert r["lo"].shape == (1, 320) and r["rs"].shape == (1, 4)
    assert np.all(np.isfinite(r["out"]))
