"""Seeded synthetic inputs for the hyper-connection read.

This module only draws numbers: it holds none of the read's arithmetic, and
it is the one piece that both the HIP path's tests/bench and the FP64
reference consume.  Weights are produced as BF16 bit patterns (``uint16``);
those bytes are what both sides read.

Every draw comes from ``numpy.random.Generator(PCG64(SeedSequence(key)))``,
where ``key`` is a tuple ``(base, purpose, index)`` so that every tensor has
its own stream and adding a tensor never shifts another one.

Shapes (token-major, contiguous):
    x, pending, out : [T][S][d]   float32
    inj             : [T][R]      float32
    w_norm          : [S][d]      float32
    w_down          : [R][S*d]    uint16 (BF16), row-major
    w_up            : [S*d][R]    uint16 (BF16), row-major
with the geometry of the pages' read, S = 4 streams of d = 2560 values and
R = 320 (Strata PR #2812, What changed: a 1,280-column slab is half a
stream, 16 columns x 4 streams are 64 rows of the up weights, K = 320).
"""

from dataclasses import dataclass

import numpy as np

S_STREAMS = 4
D_STREAM = 2560
R_DOWN = 320
T_MAX = 8       # largest verify window the pages measure
T_WIDE = 16     # larger windows, also generated

# purposes (second element of a seed key)
_P_WDOWN, _P_WUP, _P_WNORM, _P_X, _P_PENDING, _P_INJ, _P_NEARDUP, _P_EDGE, _P_MV_W, _P_MV_X = range(1, 11)


def rng(*key):
    """The generator of one seed key (a tuple of non-negative ints)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def f32_to_bf16_bits(a):
    """Round float32 values to the nearest BF16 (ties to even); return the uint16 patterns.

    Input generation only: the weights are drawn in float32 and stored as BF16.
    NaN is not expected from the draws and is not special-cased.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


@dataclass
class WeightSet:
    """One layer half's weights: BF16 down/up projections and the FP32 norm weight."""
    w_down: np.ndarray  # uint16 [R][S*d]
    w_up: np.ndarray    # uint16 [S*d][R]
    w_norm: np.ndarray  # float32 [S][d]

    @property
    def nbytes(self):
        return self.w_down.nbytes + self.w_up.nbytes + self.w_norm.nbytes


def weight_set(base, index=0, S=S_STREAMS, d=D_STREAM, R=R_DOWN):
    """W_down ~ N(0, 1/sqrt(S*d)), W_up ~ N(0, 1/sqrt(R)) (standard deviations), w_norm ~ U(0.5, 1.5)."""
    D = S * d
    wd = rng(base, _P_WDOWN, index).standard_normal((R, D), dtype=np.float32)
    wd *= np.float32(1.0 / np.sqrt(D))
    wu = rng(base, _P_WUP, index).standard_normal((D, R), dtype=np.float32)
    wu *= np.float32(1.0 / np.sqrt(R))
    wn = rng(base, _P_WNORM, index).uniform(0.5, 1.5, size=(S, d)).astype(np.float32)
    return WeightSet(f32_to_bf16_bits(wd), f32_to_bf16_bits(wu), wn)


def activations(base, T, index=0, S=S_STREAMS, d=D_STREAM):
    """x ~ N(0, 1), float32 [T][S][d]."""
    return rng(base, _P_X, index).standard_normal((T, S, d), dtype=np.float32)


def pending(base, T, index=0, S=S_STREAMS, d=D_STREAM, std=0.5):
    """The pending write, ~ N(0, std) float32 [T][S][d]."""
    p = rng(base, _P_PENDING, index).standard_normal((T, S, d), dtype=np.float32)
    return p * np.float32(std)


def injection(base, T, index=0, R=R_DOWN, std=0.1):
    """The injection added to lo, ~ N(0, std) float32 [T][R]."""
    v = rng(base, _P_INJ, index).standard_normal((T, R), dtype=np.float32)
    return v * np.float32(std)


def heavy_tailed_activations(base, T, index=0, S=S_STREAMS, d=D_STREAM,
                             nu=3.0, rms=(1e-3, 1e-1, 1e1, 1e3)):
    """Student-t(nu) draws; each (token, stream) row is scaled to a sample RMS of rms[s].

    So the per-stream RMS spans six decades across the streams of every token.
    """
    if len(rms) != S:
        raise ValueError("one target RMS per stream")
    x = rng(base, _P_X, index).standard_t(nu, size=(T, S, d))
    cur = np.sqrt(np.mean(x * x, axis=2, keepdims=True))
    x = x / cur * np.asarray(rms, dtype=np.float64)[None, :, None]
    return x.astype(np.float32)


def with_near_duplicate_rows(w_down_bits, base, index=0, frac_rows=0.01,
                             frac_entries=0.01, first_row=4):
    """Copy of w_down where round(frac_rows * R) rows are near-duplicates of other rows.

    Each chosen target row (from rows first_row..R-1) becomes a copy of a
    different, seeded source row with frac_entries of its entries moved by one
    BF16 unit in the last place (the bit pattern +1 or -1, which keeps the
    sign), so the two rows' dot products nearly tie.
    """
    w = np.array(w_down_bits, dtype=np.uint16, copy=True)
    R, D = w.shape
    g = rng(base, _P_NEARDUP, index)
    n_rows = max(1, int(round(frac_rows * R)))
    targets = g.choice(np.arange(first_row, R), size=n_rows, replace=False)
    for tr in targets:
        src = int(g.integers(0, R - 1))
        if src >= tr:
            src += 1
        row = w[src].astype(np.int32)
        n_ent = max(1, int(round(frac_entries * D)))
        cols = g.choice(D, size=n_ent, replace=False)
        step = g.choice(np.array([-1, 1]), size=n_ent)
        mag = row[cols] & 0x7FFF
        # stay inside the finite, non-zero patterns of the same sign
        step = np.where(mag <= 1, 1, np.where(mag >= 0x7F7F, -1, step))
        row[cols] = (row[cols] & 0x8000) | (mag + step)
        w[tr] = row.astype(np.uint16)
    return w, np.sort(targets)


Q8_BLOCK = 32  # weights per block of the Q8_0 copies (along a row)
Q8_EDGE_FAMILIES = ("normal", "zero", "one_nonzero", "half_integers_amax_127", "tiny", "large", "huge",
                    "negative_amax", "opposite_amax", "multiples_of_2^-7", "subnormal_scale")


def q8_edge_weights(base, rows=64, K=1024, index=0):
    """BF16 bits [rows][K] whose 32-weight blocks cycle through ``Q8_EDGE_FAMILIES``.

    Block b (row-major over the rows' blocks) has family b mod 11: N(0, 0.02);
    all zero; one nonzero entry; half-integers +-0.5 .. +-126.5 with one +-127
    (a block maximum of 127 puts every entry on a rounding tie); N(0, 1e-7);
    N(0, 1e4); N(0, 1e7); N(0, 0.02) with its largest magnitude made negative;
    two entries +A and -A as the largest magnitudes; integers -127..127 times
    2**-7 with one +-127; N(0, 1e-4) (a block maximum whose scale is a binary16
    subnormal).  Every value is drawn in float32 and stored as BF16.
    """
    if K % Q8_BLOCK:
        raise ValueError("K must be a multiple of 32")
    g = rng(base, _P_EDGE, index)
    nb = rows * K // Q8_BLOCK
    w = np.zeros((nb, Q8_BLOCK), dtype=np.float32)
    for b in range(nb):
        fam = b % len(Q8_EDGE_FAMILIES)
        z = g.standard_normal(Q8_BLOCK).astype(np.float32)
        if fam == 0:
            w[b] = 0.02 * z
        elif fam == 2:
            w[b, int(g.integers(0, Q8_BLOCK))] = np.float32(g.standard_normal() * 0.05)
        elif fam == 3:
            v = g.integers(-127, 127, size=Q8_BLOCK).astype(np.float32) + np.float32(0.5)
            v[int(g.integers(0, Q8_BLOCK))] = np.float32(127.0 if g.integers(0, 2) else -127.0)
            w[b] = v
        elif fam == 4:
            w[b] = np.float32(1e-7) * z
        elif fam == 5:
            w[b] = np.float32(1e4) * z
        elif fam == 6:
            w[b] = np.float32(1e7) * z
        elif fam == 7:
            v = 0.02 * z
            i = int(np.argmax(np.abs(v)))
            v[i] = -np.abs(v[i]) * np.float32(1.5)
            w[b] = v
        elif fam == 8:
            v = 0.01 * z
            i, j = g.choice(Q8_BLOCK, size=2, replace=False)
            a = np.float32(np.max(np.abs(v)) * 2.0 + 0.01)
            v[i], v[j] = a, -a
            w[b] = v
        elif fam == 9:
            v = g.integers(-127, 128, size=Q8_BLOCK).astype(np.float32)
            v[int(g.integers(0, Q8_BLOCK))] = np.float32(127.0 if g.integers(0, 2) else -127.0)
            w[b] = v * np.float32(2.0 ** -7)
        elif fam == 10:
            w[b] = np.float32(1e-4) * z
    return f32_to_bf16_bits(w.reshape(rows, K))


MV_ROWS, MV_COLS, MV_T_MAX = 12288, 2560, 4  # the pages' attn_q projection, 1..4 columns


def matvec_weights(base, index=0, rows=MV_ROWS, cols=MV_COLS):
    """W ~ N(0, 1/sqrt(cols)) as BF16 bits [rows][cols] (one copy of the skinny matvec's weights)."""
    w = rng(base, _P_MV_W, index).standard_normal((rows, cols), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(cols))
    return f32_to_bf16_bits(w)


def matvec_int_weights(base, rows, cols, index=0):
    """W = k / 16 with k uniform in -8..8, as BF16 bits [rows][cols] (exact in BF16; cheap to draw for very
    tall matrices)."""
    k = rng(base, _P_MV_W, index).integers(-8, 9, size=rows * cols, dtype=np.int8)
    w = k.astype(np.float32) * np.float32(0.0625)
    return (w.view(np.uint32) >> np.uint32(16)).astype(np.uint16).reshape(rows, cols)


def matvec_x(base, T, index=0, cols=MV_COLS):
    """x ~ N(0, 1), float32 [T][cols]."""
    return rng(base, _P_MV_X, index).standard_normal((T, cols), dtype=np.float32)


# ---------------------------------------------------------------------------
# The workloads.  Each returns plain numpy arrays; the caller moves them to the
# device (HIP path) or hands them to the FP64 reference.
# ---------------------------------------------------------------------------

def single_read(seed=0):
    """Real geometry, T = 1, one weight set, no pending write or injection."""
    return {"weights": [weight_set(seed, 0)], "T": 1,
            "x": activations(seed, 1), "pending": None, "inj": None}


def cold_sweep_weights(n_sets=32, base=2):
    """The rotated weight sets of the cold T sweep (32 sets, about 420 MB of BF16)."""
    return [weight_set(base, k) for k in range(n_sets)]


def cold_sweep_x(T, base=2):
    return activations(base, T, index=1000 + T)


def full_epilogue(seed=7, T=4, n_sets=32):
    """T = 4 with the pending write and the injection on; 32 rotated weight sets."""
    return {"weights": [weight_set(seed, k) for k in range(n_sets)], "T": T,
            "x": [activations(seed, T, index=k) for k in range(n_sets)],
            "pending": [pending(seed, T, index=k) for k in range(n_sets)],
            "inj": [injection(seed, T, index=k) for k in range(n_sets)]}


def verify_window(n_reads=96, T=6, base=4):
    """96 distinct weight sets (one per layer half), x_0, and one pending write per read."""
    return {"weights": [weight_set(base, k) for k in range(n_reads)], "T": T,
            "x0": activations(base, T, index=0),
            "pending": [pending(base, T, index=k) for k in range(n_reads)]}


def numerics_stress(seed=5, T=8, n_sets=32):
    """T tokens (8 by default), heavy-tailed x over six decades of stream RMS, near-tie rows, pending and inj on."""
    ws = []
    for k in range(n_sets):
        w = weight_set(seed, k)
        wd, _ = with_near_duplicate_rows(w.w_down, seed, index=k)
        ws.append(WeightSet(wd, w.w_up, w.w_norm))
    return {"weights": ws, "T": T,
            "x": [heavy_tailed_activations(seed, T, index=k) for k in range(n_sets)],
            "pending": [pending(seed, T, index=k) for k in range(n_sets)],
            "inj": [injection(seed, T, index=k) for k in range(n_sets)]}
