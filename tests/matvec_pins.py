"""Pins of the skinny BF16 matvec reference: checks against things other than the reference itself.

Each ``pin_*`` takes ``mv`` with the reference's signature ``mv(w_bits, x)``
and raises ``AssertionError`` when it disagrees with:

* exact rational arithmetic (``fractions.Fraction``) on small shapes: BF16
  weights and float32 inputs are exact binary fractions, so the exact sum is
  the ground truth, and float64 must come within its rounding bound;
* a closed form with identity-like weights (BF16 holds 0 and 1 exactly);
* ``torch.nn.functional.linear`` in float64 (a library routine);
* linearity in x and token (column) independence.
"""

from fractions import Fraction

import numpy as np
import torch
import torch.nn.functional as F

from bf16_hyper_connection_amd import inputs as gen


def _bf16_to_fraction(b):
    u = np.array([int(b) << 16], dtype=np.uint32).view(np.float32)[0]
    return Fraction(float(u))


def pin_exact_small(mv):
    for rows, cols, T, seed in ((3, 16, 1, 1), (5, 40, 3, 2), (2, 72, 4, 3)):
        w = gen.matvec_weights(seed, rows=rows, cols=cols)
        x = gen.matvec_x(seed, T, cols=cols)
        got = mv(w, x)
        assert got.shape == (T, rows)
        for t in range(T):
            for n in range(rows):
                exact = sum(_bf16_to_fraction(w[n, k]) * Fraction(float(x[t, k])) for k in range(cols))
                mag = sum(abs(_bf16_to_fraction(w[n, k]) * Fraction(float(x[t, k]))) for k in range(cols))
                err = abs(Fraction(float(got[t, n])) - exact)
                assert err <= mag * Fraction(cols + 1, 2 ** 52), (t, n, float(err), float(mag))


def pin_identity(mv):
    rows, cols, T = 24, 64, 3
    w = np.zeros((rows, cols), dtype=np.float32)
    w[np.arange(rows), (np.arange(rows) * 5) % cols] = 1.0
    w[np.arange(rows), (np.arange(rows) * 5 + 1) % cols] = -2.0
    x = gen.matvec_x(4, T, cols=cols).astype(np.float64)
    got = mv(gen.f32_to_bf16_bits(w), x)
    want = x[:, (np.arange(rows) * 5) % cols] - 2.0 * x[:, (np.arange(rows) * 5 + 1) % cols]
    assert np.array_equal(got, want)


def pin_torch_linear(mv):
    w = gen.matvec_weights(6, rows=300, cols=512)
    x = gen.matvec_x(6, 4, cols=512)
    wt = torch.from_numpy(w.astype(np.int16)).view(torch.bfloat16).to(torch.float64)
    ref = F.linear(torch.from_numpy(x.astype(np.float64)), wt).numpy()
    got = mv(w, x)
    assert np.max(np.abs(got - ref)) <= 1e-13 * np.max(np.abs(ref))


def pin_linearity_and_columns(mv):
    w = gen.matvec_weights(7, rows=64, cols=256)
    x = gen.matvec_x(7, 4, cols=256).astype(np.float64)
    y = mv(w, x)
    y2 = mv(w, 2.0 * x)
    assert np.array_equal(y2, 2.0 * y)                       # scaling by 2 is exact
    for t in range(4):
        assert np.allclose(mv(w, x[t:t + 1])[0], y[t], rtol=1e-14, atol=1e-14)
    # W then a row permutation: the outputs permute the same way
    perm = np.random.default_rng(7).permutation(64)
    assert np.array_equal(mv(w[perm], x), y[:, perm])


ALL_PINS = [pin_exact_small, pin_identity, pin_torch_linear, pin_linearity_and_columns]
