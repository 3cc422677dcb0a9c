"""FP64 CPU reference ("oracle") of the BF16 hyper-connection read, its Q8_0 sibling and the skinny BF16 matvec.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in this
package. The product path (``bf16_hyper_connection_amd``) never imports it,
and the two share no code: no kernels, headers, helpers, tables or constants.
"""

from .reference import (  # noqa: F401
    EPS,
    bf16_bits_to_f64,
    down_projection,
    epilogue,
    hc_read,
    hc_read_decoded,
    stream_rms_scale,
    up_projection,
)
from .q8_0 import dequantize_q8_0, hc_read_q8_0, quantize_q8_0  # noqa: F401,E402
from .matvec import matvec_bf16  # noqa: F401,E402
