"""TurboQuant KV-cache compression and compressed decode attention for MI355X.

The work is done by the HIP library libtq.so (C ABI in include/tq.h); this
package only builds it (build.py) and binds it (binding.py).
"""
from . import binding  # noqa: F401
from .binding import (TQ_F16, TQ_F32, TQ_KEYS, TQ_ROT_HAAR, TQ_ROT_HADAMARD, TQ_VALUES,  # noqa: F401
                      Cache, Layer, TQError, attn_decode, dequantize, get_codebook, host_tables,
                      make_rotation, quantize_kv)
