"""FP64 CPU reference of the BF16 hyper-connection (HC) read.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. It shares
no code with the HIP path and imports nothing from it.

What the pages fix, and what this module reads into them
--------------------------------------------------------
Strata PR #2812 ("sycl: STRATA_GR_FUSED=1, the two-kernel BF16
hyper-connection read (opt-in)"), sections Summary and What changed, and
Strata PR #2070 (Turing kernels for the hyper-connection read), first
comment, describe the read per token of a speculative-decode verify window:
the residual streams are normalised by a per-stream RMS scale ``rs`` (the
"norm"), a down projection of the 4 x 2560 stream values to 320 values
``lo`` follows (the injection, when present, is written with ``lo``), then an
up projection from 320 back to 4 x 2560, and an epilogue made of the pending
write, a gate and the stream mean.  The down kernel stages the weighted
streams unscaled together with their sums of squares, and applies ``rs``
per stream only when it finishes the split reduction; this module applies
the same factor after the dot product, which is the same quantity.

The pages give the structure, not the formulas, and print no worked
example.  The plainest reading that the rest supports, taken here, per
token ``t``, stream ``s`` (0..S-1), stream column ``c`` (0..d-1), down row
``r`` (0..R-1) and up row ``j = s*d + c``:

    rs[t,s]    = 1 / sqrt( (1/d) * sum_c x[t,s,c]^2 + eps ),  eps = 1e-6
    lo[t,r]    = sum_s rs[t,s] * sum_c W_down[r, s*d+c] * x[t,s,c] * w_norm[s,c]
                 + inj[t,r]                                   (inj optional)
    u[t,j]     = sum_k W_up[j,k] * lo[t,k]
    out[t,s,c] = pending[t,s,c] (optional, else 0) + sigmoid(lo[t,s]) * u[t,s*d+c]
    mean[t,c]  = (1/S) * sum_s out[t,s,c]

Weights are BF16 bit patterns (``uint16``); everything else is decoded to
float64 exactly and computed in float64.  No step is blocked, fused or
reordered beyond what these formulas state; ``@`` (a float64 matrix product)
is the only library primitive used.  Every function is pinned by the CPU
tests (brute force in 50-digit arithmetic on small shapes, closed forms with
identity-like weights, the library RMSNorm and linear routines, and the
gate/mean/scale/token invariants).  Agreement with the pages' own numerics
cannot be pinned: they print no values.
"""

import numpy as np

EPS = 1e-6  # added to the mean of squares, inside the square root


def bf16_bits_to_f64(bits):
    """Decode BF16 bit patterns (uint16 array) to float64, exactly.

    A bfloat16 value is the upper half of an IEEE binary32 word, so the
    pattern shifted left by 16 bits is the float32 of the same value.
    """
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def stream_rms_scale(x, eps=EPS):
    """rs[t,s] = 1/sqrt(mean_c x[t,s,c]^2 + eps): the per-stream RMS scale.

    The scale that the work-group finishing the down reduction multiplies
    into each stream's partial sums (Strata PR #2812, What changed), taken
    over the raw stream values whose sums of squares the down kernel stages.
    x: [T][S][d].  Returns [T][S] float64.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=2)
    return 1.0 / np.sqrt(ms + eps)


def down_projection(x, w_norm, w_down, rs, inj=None):
    """lo[t,r] = sum_s rs[t,s] * (W_down[:, s-th column block] . (x[t,s] * w_norm[s])) + inj[t,r].

    The down projection from the 4 x 2560 normalised stream values to 320
    (Strata PR #2812, Summary and What changed).  Column block s of W_down
    (columns s*d .. s*d+d-1) multiplies stream s.
    x: [T][S][d], w_norm: [S][d], w_down: [R][S*d] float64, rs: [T][S],
    inj: [T][R] or None.  Returns lo [T][R] float64.
    """
    x = np.asarray(x, dtype=np.float64)
    w_norm = np.asarray(w_norm, dtype=np.float64)
    T, S, d = x.shape
    R = w_down.shape[0]
    lo = np.zeros((T, R), dtype=np.float64)
    for t in range(T):
        for s in range(S):
            staged = x[t, s] * w_norm[s]               # unscaled, as the kernel stages it
            dot = w_down[:, s * d:(s + 1) * d] @ staged
            lo[t] += rs[t, s] * dot
    if inj is not None:
        lo += np.asarray(inj, dtype=np.float64)
    return lo


def up_projection(lo, w_up):
    """u[t,j] = sum_k W_up[j,k] * lo[t,k]: the up projection from 320 to 4 x 2560.

    Strata PR #2812, What changed (the up kernel reduces over K = 320).
    lo: [T][R], w_up: [S*d][R] float64.  Returns u [T][S*d] float64.
    """
    lo = np.asarray(lo, dtype=np.float64)
    return lo @ w_up.T


def epilogue(lo, u, S, pending=None):
    """out = pending + sigmoid(lo[t,s]) * u (stream s); mean = average of out over streams.

    The up kernel's epilogue (Strata PR #2812, What changed: pending write,
    gate, stream mean).  The gate of stream s is the logistic sigmoid of
    lo[t,s], after the injection.
    lo: [T][R], u: [T][S*d], pending: [T][S][d] or None.
    Returns out [T][S][d] and mean [T][d], float64.
    """
    T = lo.shape[0]
    d = u.shape[1] // S
    u = u.reshape(T, S, d)
    gate = 1.0 / (1.0 + np.exp(-lo[:, :S]))             # [T][S]
    out = gate[:, :, None] * u
    if pending is not None:
        out = out + np.asarray(pending, dtype=np.float64)
    mean = np.sum(out, axis=1) / S
    return out, mean


def hc_read(x, w_norm, w_down_bits, w_up_bits, pending=None, inj=None, eps=EPS):
    """One HC read for T tokens: norm, down, up and epilogue, all in float64.

    x: [T][S][d] (any float dtype), w_norm: [S][d], w_down_bits: uint16 [R][S*d],
    w_up_bits: uint16 [S*d][R], pending: [T][S][d] or None, inj: [T][R] or None.
    Returns a dict with out [T][S][d], mean [T][d], lo [T][R], rs [T][S], u [T][S*d].
    """
    return hc_read_decoded(x, w_norm, bf16_bits_to_f64(w_down_bits), bf16_bits_to_f64(w_up_bits),
                           pending=pending, inj=inj, eps=eps)


def hc_read_decoded(x, w_norm, w_down, w_up, pending=None, inj=None, eps=EPS):
    """The same read on weights already decoded to float64 (any storage format).

    w_down: [R][S*d] float64, w_up: [S*d][R] float64; the rest as ``hc_read``.
    """
    x = np.asarray(x, dtype=np.float64)
    T, S, d = x.shape
    R = w_down.shape[0]
    if w_down.shape != (R, S * d) or w_up.shape != (S * d, R):
        raise ValueError("weight shapes do not match x")
    if R < S:
        raise ValueError("the gate needs lo[0..S-1], so R >= S")
    rs = stream_rms_scale(x, eps)
    lo = down_projection(x, w_norm, w_down, rs, inj)
    u = up_projection(lo, w_up)
    out, mean = epilogue(lo, u, S, pending)
    return {"out": out, "mean": mean, "lo": lo, "rs": rs, "u": u}
