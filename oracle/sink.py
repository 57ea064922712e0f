"""Decode with an fp16 attention-sink segment (oracle).

Test infrastructure only (see ``oracle/__init__.py``).

Source: the unite.ai axis-selection guide, future-directions section: besides
the window of recently generated tokens, a high-precision window is kept for
the attention-sink tokens (InnerQ), so that no outlier channel of theirs
spoils a quantized group.  The pages give no more than that; the reading
taken: the sink is the sequence's first n_sink tokens, kept in fp16 and never
quantized; the cache holds the tokens after them (quantized, then the fp16
window); the decode attends over the sink, then the quantized tokens, then
the window.  Without a rotary embedding positions play no part, so the order
of the three segments does not change the result.  With keys stored before
the rotary embedding (``rope``), the token order fixes the positions: sink
token s at position s, then the cache's tokens from position S on.
"""

import numpy as np

from .attention import attention
from .cache import context
from .rope import rope


def decode_head_sink(q, state, sink_k, sink_v, alpha, group, bits, rope_base=None):
    """Decode output (fp64 [D]) of one (sequence, head): fp16 sink rows
    sink_k, sink_v [S, D] (S may be 0) followed by the cache state's
    dequantized context.  With ``rope_base``, every key (stored before the
    rotation) is rotated by its position in that order; q is the rotated
    query."""
    kk, vv = context(state, group, bits)
    sk = np.asarray(sink_k, dtype=np.float64).reshape(-1, kk.shape[1])
    sv = np.asarray(sink_v, dtype=np.float64).reshape(-1, vv.shape[1])
    keys = np.concatenate([sk, kk])
    if rope_base is not None:
        keys = rope(keys, np.arange(keys.shape[0]), rope_base)
    return attention(q, keys, np.concatenate([sv, vv]), alpha)
