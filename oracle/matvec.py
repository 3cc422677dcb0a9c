"""FP64 CPU reference of the skinny BF16 matrix-vector product.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. It shares
no code with the HIP path and imports nothing from it.

Strata PR #2221 (the Turing Q2_0 matvec with four rows per warp, first
comment) measures the decode-window projection attn_q, 2,560 inputs to
12,288 outputs, at one to four columns (the window's tokens), with cold
weights.  Its Q2_0 format is not defined on the pages, so the workload here
keeps the shape and the access pattern with BF16 weights, the format of the
rest of this library.  Per column t and output row n:

    y[t, n] = sum_k W[n, k] * x[t, k]

W: BF16 bit patterns [N][K] (uint16), row-major; x: [T][K]; y: [T][N].
Decoded exactly to float64 and computed in float64 with ``@`` (the one
library primitive used).
"""

import numpy as np

from .reference import bf16_bits_to_f64


def matvec_bf16(w_bits, x):
    """y[t, n] = sum_k W[n, k] x[t, k] in float64.  w_bits: uint16 [N][K]; x: [T][K].  Returns [T][N]."""
    w = bf16_bits_to_f64(w_bits)
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("x must be [T][K] with K = the columns of W")
    return x @ w.T
