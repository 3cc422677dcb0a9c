"""Planted mistakes in copies of the FP64 reference must each fail at least one pin.

Every mutant below is the reference with one plausible slip (a dropped term,
a wrong sign, index or axis, a transposed operand); the mistake is planted in
a CPU copy of the reference, never in the HIP path.
"""

import numpy as np
import pytest

import oracle
from oracle import reference as ref
from tests import oracle_pins as pins


def _read_with(**overrides):
    """A copy of the reference read with some of its steps replaced."""
    steps = {"rs": ref.stream_rms_scale, "down": ref.down_projection,
             "up": ref.up_projection, "epi": ref.epilogue}
    steps.update(overrides)

    def read(x, w_norm, w_down_bits, w_up_bits, pending=None, inj=None):
        x = np.asarray(x, dtype=np.float64)
        T, S, d = x.shape
        wd = oracle.bf16_bits_to_f64(w_down_bits)
        wu = oracle.bf16_bits_to_f64(w_up_bits)
        rs = steps["rs"](x)
        lo = steps["down"](x, w_norm, wd, rs, inj)
        u = steps["up"](lo, wu)
        out, mean = steps["epi"](lo, u, S, pending)
        return {"out": out, "mean": mean, "lo": lo, "rs": rs, "u": u}
    return read


def _rs_eps_outside(x, eps=ref.EPS):
    return 1.0 / (np.sqrt(np.mean(x * x, axis=2)) + eps)


def _rs_sum_not_mean(x, eps=ref.EPS):
    return 1.0 / np.sqrt(np.sum(x * x, axis=2) + eps)


def _rs_per_token(x, eps=ref.EPS):
    ms = np.mean(x * x, axis=(1, 2))
    return np.repeat((1.0 / np.sqrt(ms + eps))[:, None], x.shape[1], axis=1)


def _rs_no_eps(x, eps=ref.EPS):
    return 1.0 / np.sqrt(np.mean(x * x, axis=2))


def _down_no_wnorm(x, w_norm, w_down, rs, inj=None):
    return ref.down_projection(x, np.ones_like(np.asarray(w_norm, dtype=np.float64)), w_down, rs, inj)


def _down_no_inj(x, w_norm, w_down, rs, inj=None):
    return ref.down_projection(x, w_norm, w_down, rs, None)


def _down_reversed_blocks(x, w_norm, w_down, rs, inj=None):
    T, S, d = x.shape
    wd = np.concatenate([w_down[:, s * d:(s + 1) * d] for s in reversed(range(S))], axis=1)
    return ref.down_projection(x, w_norm, wd, rs, inj)


def _down_rs_squared(x, w_norm, w_down, rs, inj=None):
    return ref.down_projection(x, w_norm, w_down, rs * rs, inj)


def _down_interleaved_columns(x, w_norm, w_down, rs, inj=None):
    # reads column j = c*S + s instead of s*d + c
    T, S, d = x.shape
    wd = w_down.reshape(w_down.shape[0], d, S).transpose(0, 2, 1).reshape(w_down.shape[0], S * d)
    return ref.down_projection(x, w_norm, wd, rs, inj)


def _up_transposed(lo, w_up):
    return lo @ w_up.reshape(w_up.shape[1], w_up.shape[0])


def _epi_gate_wrong_rows(lo, u, S, pending=None):
    return ref.epilogue(np.roll(lo, -S, axis=1), u, S, pending) if lo.shape[1] >= 2 * S else \
        ref.epilogue(np.roll(lo, -1, axis=1), u, S, pending)


def _epi_gate_sign(lo, u, S, pending=None):
    T = lo.shape[0]
    d = u.shape[1] // S
    gate = 1.0 / (1.0 + np.exp(lo[:, :S]))
    out = gate[:, :, None] * u.reshape(T, S, d)
    if pending is not None:
        out = out + pending
    return out, out.mean(axis=1)


def _epi_no_pending(lo, u, S, pending=None):
    return ref.epilogue(lo, u, S, None)


def _epi_mean_wrong_divisor(lo, u, S, pending=None):
    out, mean = ref.epilogue(lo, u, S, pending)
    return out, mean * S / max(S - 1, 1)


def _epi_interleaved_rows(lo, u, S, pending=None):
    # reads up row j = c*S + s instead of s*d + c
    T = lo.shape[0]
    d = u.shape[1] // S
    u2 = u.reshape(T, d, S).transpose(0, 2, 1).reshape(T, S * d)
    return ref.epilogue(lo, u2, S, pending)


def _epi_gate_before_inj(lo, u, S, pending=None):
    # gate computed from lo with the token mean removed (a stand-in for "before the injection")
    return ref.epilogue(lo - lo.mean(axis=1, keepdims=True), u, S, pending)


MUTANTS = {
    "rs_eps_outside_sqrt": dict(rs=_rs_eps_outside),
    "rs_sum_not_mean": dict(rs=_rs_sum_not_mean),
    "rs_per_token": dict(rs=_rs_per_token),
    "rs_no_eps": dict(rs=_rs_no_eps),
    "down_no_w_norm": dict(down=_down_no_wnorm),
    "down_drops_injection": dict(down=_down_no_inj),
    "down_stream_blocks_reversed": dict(down=_down_reversed_blocks),
    "down_rs_squared": dict(down=_down_rs_squared),
    "down_columns_interleaved": dict(down=_down_interleaved_columns),
    "up_transposed": dict(up=_up_transposed),
    "gate_wrong_rows": dict(epi=_epi_gate_wrong_rows),
    "gate_sign_flipped": dict(epi=_epi_gate_sign),
    "pending_dropped": dict(epi=_epi_no_pending),
    "mean_wrong_divisor": dict(epi=_epi_mean_wrong_divisor),
    "up_rows_interleaved": dict(epi=_epi_interleaved_rows),
    "gate_shifted_input": dict(epi=_epi_gate_before_inj),
}


def test_unmutated_copy_passes_every_pin():
    read = _read_with()
    for pin in pins.ALL_PINS:
        pin(read)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name):
    read = _read_with(**MUTANTS[name])
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(read)
        except (AssertionError, ValueError) as e:  # noqa: PERF203
            failed.append((pin.__name__, str(e)[:80]))
    assert failed, f"mutant {name} passed every pin"
