"""Pins of the FP64 reference: checks against things other than the reference itself.

Each ``pin_*`` takes ``read``, a function with the reference's signature
``read(x, w_norm, w_down_bits, w_up_bits, pending=None, inj=None)`` that
returns a dict with ``out``, ``mean``, ``lo`` and ``rs``, and raises
``AssertionError`` when ``read`` disagrees with:

* brute force in 50-digit arithmetic on small shapes (mpmath);
* closed forms with identity-like weights (exactly representable in BF16);
* library routines: ``torch.nn.functional.rms_norm`` and ``linear`` in float64;
* invariants: a saturated gate, a zero stream, per-stream scale invariance,
  token independence and the stream mean.

The pages print no worked example, so these are the pins (there are no
stored values from the pages).  ``tests/test_oracle.py`` runs them on the
reference; ``tests/test_oracle_mutants.py`` runs them on copies of the
reference with planted mistakes and requires each copy to fail one of them.
"""

import math

import mpmath
import numpy as np
import torch
import torch.nn.functional as F

from bf16_hyper_connection_amd import inputs as gen

EPS = 1e-6


def _bits_to_f64(bits):
    # independent of the reference's decoder: via torch's bfloat16 type
    t = torch.from_numpy(np.asarray(bits, dtype=np.uint16).astype(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def _small_case(S, d, R, T, seed, with_pending=True, with_inj=True):
    w = gen.weight_set(seed, 0, S=S, d=d, R=R)
    x = gen.activations(seed, T, S=S, d=d)
    p = gen.pending(seed, T, S=S, d=d) if with_pending else None
    inj = gen.injection(seed, T, R=R) if with_inj else None
    return w, x, p, inj


def _rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale)


# ---------------------------------------------------------------------------
# brute force
# ---------------------------------------------------------------------------

def brute_force_read(x, w_norm, w_down_bits, w_up_bits, pending, inj, dps=50):
    """The read's definition as scalar loops in mpmath at ``dps`` digits."""
    mp = mpmath.mp.clone()
    mp.dps = dps
    T, S, d = x.shape
    wd = _bits_to_f64(w_down_bits)
    wu = _bits_to_f64(w_up_bits)
    R = wd.shape[0]
    f = lambda v: mp.mpf(float(v))  # noqa: E731  (exact: binary64 -> mpf)
    res = {"out": np.zeros((T, S, d)), "mean": np.zeros((T, d)),
           "lo": np.zeros((T, R)), "rs": np.zeros((T, S))}
    for t in range(T):
        rs = []
        for s in range(S):
            acc = mp.mpf(0)
            for c in range(d):
                acc += f(x[t, s, c]) ** 2
            rs.append(1 / mp.sqrt(acc / d + f(EPS)))
            res["rs"][t, s] = float(rs[-1])
        lo = []
        for r in range(R):
            acc = mp.mpf(0)
            for s in range(S):
                part = mp.mpf(0)
                for c in range(d):
                    part += f(wd[r, s * d + c]) * f(x[t, s, c]) * f(w_norm[s, c])
                acc += rs[s] * part
            if inj is not None:
                acc += f(inj[t, r])
            lo.append(acc)
            res["lo"][t, r] = float(acc)
        outs = [[None] * d for _ in range(S)]
        for s in range(S):
            gate = 1 / (1 + mp.exp(-lo[s]))
            for c in range(d):
                u = mp.mpf(0)
                for k in range(R):
                    u += f(wu[s * d + c, k]) * lo[k]
                o = gate * u + (f(pending[t, s, c]) if pending is not None else 0)
                outs[s][c] = o
                res["out"][t, s, c] = float(o)
        for c in range(d):
            acc = mp.mpf(0)
            for s in range(S):
                acc += outs[s][c]
            res["mean"][t, c] = float(acc / S)
    return res


def pin_brute_force(read, shapes=((4, 8, 6, 3), (2, 5, 3, 2), (4, 16, 8, 1)), seed=11):
    for (S, d, R, T) in shapes:
        for wp, wi in ((True, True), (False, False), (True, False)):
            w, x, p, inj = _small_case(S, d, R, T, seed, wp, wi)
            got = read(x, w.w_norm, w.w_down, w.w_up, pending=p, inj=inj)
            ref = brute_force_read(x, w.w_norm, w.w_down, w.w_up, p, inj)
            for key in ("out", "mean", "lo", "rs"):
                e = _rel_err(got[key], ref[key])
                assert e <= 1e-13, f"brute force {key} S={S} d={d} R={R} T={T}: rel err {e:.3e}"


# ---------------------------------------------------------------------------
# closed forms with identity-like weights
# ---------------------------------------------------------------------------

def closed_form_case(S, d, R, T, seed=3):
    """Identity-like weights (0, 1, 2, 3, 4 are exact in BF16) and constant streams.

    W_down[r, s*d + c] = (s + 1) * [c == r]      (needs R <= d)
    W_up[s*d + c, k]   = [k == (c + s) mod R]
    x[t, s, c]         = a[t, s]  (a constant per stream)
    Then, with m = 1e-6:
      rs[t,s]    = 1 / sqrt(a[t,s]^2 + m)
      lo[t,r]    = sum_s (s+1) * rs[t,s] * a[t,s] * w_norm[s,r] + inj[t,r]
      u[t,s,c]   = lo[t, (c+s) mod R]
      out[t,s,c] = pending[t,s,c] + sigmoid(lo[t,s]) * lo[t,(c+s) mod R]
    """
    assert R <= d and S <= R
    D = S * d
    wd = np.zeros((R, D), dtype=np.uint16)
    for s in range(S):
        for r in range(R):
            wd[r, s * d + r] = gen.f32_to_bf16_bits(np.array([s + 1], dtype=np.float32))[0]
    wu = np.zeros((D, R), dtype=np.uint16)
    one = gen.f32_to_bf16_bits(np.array([1.0], dtype=np.float32))[0]
    for s in range(S):
        for c in range(d):
            wu[s * d + c, (c + s) % R] = one
    g = gen.rng(seed, 99, 0)
    a = g.choice(np.array([0.25, -0.5, 1.0, -2.0, 3.0, 0.125, -1.5], dtype=np.float32), size=(T, S))
    x = np.repeat(a[:, :, None], d, axis=2).astype(np.float32)
    w_norm = g.uniform(0.5, 1.5, size=(S, d)).astype(np.float32)
    pending = g.standard_normal((T, S, d)).astype(np.float32)
    inj = (0.1 * g.standard_normal((T, R))).astype(np.float32)

    rs = np.zeros((T, S))
    lo = np.zeros((T, R))
    out = np.zeros((T, S, d))
    mean = np.zeros((T, d))
    for t in range(T):
        for s in range(S):
            av = float(a[t, s])
            rs[t, s] = 1.0 / math.sqrt(av * av + EPS)
        for r in range(R):
            lo[t, r] = math.fsum((s + 1) * rs[t, s] * float(a[t, s]) * float(w_norm[s, r])
                                 for s in range(S)) + float(inj[t, r])
        for s in range(S):
            gate = 1.0 / (1.0 + math.exp(-lo[t, s]))
            for c in range(d):
                out[t, s, c] = float(pending[t, s, c]) + gate * lo[t, (c + s) % R]
        for c in range(d):
            mean[t, c] = math.fsum(out[t, s, c] for s in range(S)) / S
    return (x, w_norm, wd, wu, pending, inj), {"rs": rs, "lo": lo, "out": out, "mean": mean}


def pin_closed_form(read, shapes=((4, 16, 8, 2), (3, 7, 5, 3))):
    for (S, d, R, T) in shapes:
        (x, wn, wd, wu, p, inj), ref = closed_form_case(S, d, R, T)
        got = read(x, wn, wd, wu, pending=p, inj=inj)
        for key in ("rs", "lo", "out", "mean"):
            e = _rel_err(got[key], ref[key])
            assert e <= 1e-12, f"closed form {key} S={S} d={d} R={R}: rel err {e:.3e}"


# ---------------------------------------------------------------------------
# library routines
# ---------------------------------------------------------------------------

def pin_library_routines(read, S=4, d=32, R=12, T=3, seed=21):
    """rs*x*w_norm equals torch's RMSNorm; lo and u equal torch's linear of it."""
    w, x, p, inj = _small_case(S, d, R, T, seed)
    got = read(x, w.w_norm, w.w_down, w.w_up, pending=p, inj=inj)
    xt = torch.from_numpy(x.astype(np.float64))
    normed = torch.stack([
        torch.stack([F.rms_norm(xt[t, s], (d,), torch.from_numpy(w.w_norm[s].astype(np.float64)), eps=EPS)
                     for s in range(S)]) for t in range(T)])          # [T][S][d]
    mine = torch.from_numpy(got["rs"])[:, :, None] * xt * torch.from_numpy(w.w_norm.astype(np.float64))[None]
    e = _rel_err(mine.numpy(), normed.numpy())
    assert e <= 1e-14, f"rs*x*w_norm vs rms_norm: {e:.3e}"
    wd = torch.from_numpy(_bits_to_f64(w.w_down))
    wu = torch.from_numpy(_bits_to_f64(w.w_up))
    lo = F.linear(normed.reshape(T, S * d), wd) + torch.from_numpy(inj.astype(np.float64))
    e = _rel_err(got["lo"], lo.numpy())
    assert e <= 1e-13, f"lo vs linear(rms_norm): {e:.3e}"
    u = F.linear(lo, wu).reshape(T, S, d)
    gate = torch.sigmoid(lo[:, :S])
    out = torch.from_numpy(p.astype(np.float64)) + gate[:, :, None] * u
    e = _rel_err(got["out"], out.numpy())
    assert e <= 1e-13, f"out vs library composition: {e:.3e}"
    e = _rel_err(got["mean"], out.mean(dim=1).numpy())
    assert e <= 1e-13, f"mean vs library composition: {e:.3e}"


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def pin_gate_saturated(read, S=4, d=24, R=10, T=2, seed=31):
    """inj[:, :S] = +100: gate 1 (in fp64), out = u, mean = average of u.

    inj[:, :S] = -100: gate ~ 3.7e-44, out = pending, mean = average of pending.
    """
    w, x, p, inj = _small_case(S, d, R, T, seed)
    wu = torch.from_numpy(_bits_to_f64(w.w_up))
    inj_open = inj.copy()
    inj_open[:, :S] = 100.0
    got = read(x, w.w_norm, w.w_down, w.w_up, pending=None, inj=inj_open)
    u = F.linear(torch.from_numpy(got["lo"]), wu).reshape(T, S, d).numpy()
    assert _rel_err(got["out"], u) <= 1e-14, "open gate: out != u"
    assert _rel_err(got["mean"], u.sum(axis=1) / S) <= 1e-14, "open gate: mean != average of u"
    inj_shut = inj.copy()
    inj_shut[:, :S] = -100.0
    got = read(x, w.w_norm, w.w_down, w.w_up, pending=p, inj=inj_shut)
    pf = p.astype(np.float64)
    assert _rel_err(got["out"], pf) <= 1e-35, "shut gate: out != pending"
    assert _rel_err(got["mean"], pf.sum(axis=1) / S) <= 1e-15, "shut gate: mean != average of pending"


def pin_zero_stream(read, S=4, d=20, R=9, T=2, seed=41):
    """A zero stream has rs = 1/sqrt(1e-6) and adds nothing to lo."""
    w, x, p, inj = _small_case(S, d, R, T, seed)
    x = x.copy()
    x[:, 2, :] = 0.0
    got = read(x, w.w_norm, w.w_down, w.w_up, pending=p, inj=inj)
    assert np.allclose(got["rs"][:, 2], 1.0 / math.sqrt(EPS), rtol=1e-15, atol=0)
    wd = np.array(w.w_down, copy=True)
    wd[:, 2 * d:3 * d] = 0
    got2 = read(x, w.w_norm, wd, w.w_up, pending=p, inj=inj)
    assert _rel_err(got["lo"], got2["lo"]) <= 1e-15, "zero stream changed lo"


def pin_scale_invariance(read, S=4, d=64, R=12, T=2, seed=51):
    """Scaling stream s by c_s > 0 leaves lo (hence out) unchanged up to the eps term.

    With mean(x^2) ~ 1 and c_s in [0.1, 10], the relative change of rs*x is at
    most about eps/(2 * min(c_s^2) * mean(x^2)) ~ 5e-5.
    """
    w, x, p, inj = _small_case(S, d, R, T, seed)
    c = np.array([10.0, 0.1, 3.0, 0.5][:S], dtype=np.float32)
    got = read(x, w.w_norm, w.w_down, w.w_up, pending=p, inj=inj)
    got2 = read(x * c[None, :, None], w.w_norm, w.w_down, w.w_up, pending=p, inj=inj)
    e = _rel_err(got2["lo"], got["lo"])
    assert e <= 1e-4, f"per-stream scale changed lo by {e:.3e}"
    e = _rel_err(got2["out"], got["out"])
    assert e <= 1e-4, f"per-stream scale changed out by {e:.3e}"
    # and a single stream scaled is not the same as the token scaled: rs is per stream
    assert np.allclose(got2["rs"] * c[None, :], got["rs"], rtol=1e-3)


def pin_token_independence(read, S=4, d=16, R=8, T=4, seed=61):
    """Each token's result depends on that token's inputs only."""
    w, x, p, inj = _small_case(S, d, R, T, seed)
    got = read(x, w.w_norm, w.w_down, w.w_up, pending=p, inj=inj)
    for t in range(T):
        one = read(x[t:t + 1], w.w_norm, w.w_down, w.w_up, pending=p[t:t + 1], inj=inj[t:t + 1])
        for key in ("out", "mean", "lo", "rs"):
            e = _rel_err(one[key][0], got[key][t])
            assert e <= 1e-14, f"token {t} {key} depends on other tokens ({e:.3e})"


def pin_stream_mean(read, S=4, d=16, R=8, T=2, seed=71):
    w, x, p, inj = _small_case(S, d, R, T, seed)
    got = read(x, w.w_norm, w.w_down, w.w_up, pending=p, inj=inj)
    assert _rel_err(got["mean"], np.mean(got["out"], axis=1)) <= 1e-15


ALL_PINS = [pin_brute_force, pin_closed_form, pin_library_routines, pin_gate_saturated,
            pin_zero_stream, pin_scale_invariance, pin_token_independence, pin_stream_mean]
