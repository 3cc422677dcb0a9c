"""The seeded input generator: determinism, shapes, and the stated distributions (CPU only)."""

import numpy as np
import torch

from bf16_hyper_connection_amd import inputs as gen


def test_bf16_rounding_matches_torch():
    g = gen.rng(1, 2, 3)
    a = np.concatenate([g.standard_normal(100000).astype(np.float32) * 10.0 ** g.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0], dtype=np.float32)]).astype(np.float32)
    mine = gen.f32_to_bf16_bits(a)
    theirs = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, theirs)


def test_deterministic_and_distinct():
    a = gen.weight_set(2, 0, S=4, d=64, R=16)
    b = gen.weight_set(2, 0, S=4, d=64, R=16)
    c = gen.weight_set(2, 1, S=4, d=64, R=16)
    assert np.array_equal(a.w_down, b.w_down) and np.array_equal(a.w_up, b.w_up)
    assert not np.array_equal(a.w_down, c.w_down)
    assert np.array_equal(gen.activations(5, 3), gen.activations(5, 3))


def test_real_geometry_shapes_and_scales():
    w = gen.weight_set(0, 0)
    assert w.w_down.shape == (320, 10240) and w.w_down.dtype == np.uint16
    assert w.w_up.shape == (10240, 320) and w.w_up.dtype == np.uint16
    assert w.w_norm.shape == (4, 2560) and w.w_norm.dtype == np.float32
    assert w.w_down.nbytes + w.w_up.nbytes == 13107200
    wd = torch.from_numpy(w.w_down.view(np.int16)).view(torch.bfloat16).float().numpy()
    wu = torch.from_numpy(w.w_up.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert abs(wd.std() * np.sqrt(10240) - 1) < 0.01
    assert abs(wu.std() * np.sqrt(320) - 1) < 0.01
    assert 0.5 <= w.w_norm.min() and w.w_norm.max() <= 1.5
    x = gen.activations(0, 8)
    assert x.shape == (8, 4, 2560) and x.dtype == np.float32


def test_heavy_tailed_rms_spans_six_decades():
    x = gen.heavy_tailed_activations(5, 8)
    rms = np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=2))
    assert np.allclose(rms, np.array([1e-3, 1e-1, 1e1, 1e3])[None, :], rtol=1e-5)


def test_near_duplicate_rows():
    w = gen.weight_set(5, 0)
    wd, targets = gen.with_near_duplicate_rows(w.w_down, 5)
    assert len(targets) == 3 and targets.min() >= 4
    changed = np.nonzero(np.any(wd != w.w_down, axis=1))[0]
    assert np.array_equal(changed, targets)
    for tr in targets:
        # a near duplicate of some other row: 1 % of entries 1 ulp apart, same signs
        diffs = np.count_nonzero(wd[tr][None, :] != w.w_down, axis=1)
        src = int(np.argmin(np.where(np.arange(320) == tr, 10 ** 9, diffs)))
        assert diffs[src] == round(0.01 * 10240)
        delta = wd[tr].astype(np.int32) - w.w_down[src].astype(np.int32)
        assert set(np.unique(np.abs(delta))) <= {0, 1}
        assert np.array_equal(wd[tr] & 0x8000, w.w_down[src] & 0x8000)


def test_q8_edge_weights_are_seeded_and_cover_every_family():
    a, b = gen.q8_edge_weights(3), gen.q8_edge_weights(3)
    assert np.array_equal(a, b) and a.dtype == np.uint16 and a.shape == (64, 1024)
    blocks = a.reshape(-1, 32)
    n = len(gen.Q8_EDGE_FAMILIES)
    assert not np.any(blocks[1::n])                               # the all-zero family
    assert np.all(np.count_nonzero(blocks[2::n], axis=1) == 1)   # one nonzero entry
    assert not np.array_equal(a, gen.q8_edge_weights(4))


def test_matvec_int_weights_exact_in_bf16():
    w = gen.matvec_int_weights(3, 10, 16)
    f = (w.astype(np.uint32) << 16).view(np.float32)
    assert w.shape == (10, 16) and np.all(np.abs(f) <= 0.5) and np.all(f * 16 == np.round(f * 16))
    assert np.array_equal(w, gen.matvec_int_weights(3, 10, 16))
