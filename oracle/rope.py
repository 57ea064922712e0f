"""Rotary position embedding applied after dequantization (oracle).

Test infrastructure only (see ``oracle/__init__.py``).

Source: the unite.ai axis-selection guide, section on rotary embeddings: RoPE
rotates pairs of channels by an angle that grows with the token's position,
which mixes an outlier channel into its partner and so spoils per-channel key
groups; the remedy it describes (from KVQuant) is to quantize keys before the
rotation and rotate them after dequantization.  Its list of things to do
repeats this as a correctness matter.

The pages give no formula, so the rotation is the original rotary embedding
(RoFormer): for a head of D channels, channel pair f = (2f, 2f + 1),
f = 0 .. D/2 - 1, turns by the angle ``p * theta_f`` at position p, with
``theta_f = base ** (-2 f / D)``:

    y[2f]     = x[2f] cos(p theta_f) - x[2f+1] sin(p theta_f)
    y[2f + 1] = x[2f] sin(p theta_f) + x[2f+1] cos(p theta_f)

A head stored in the "rotate half" pairing (f, f + D/2) maps onto this one by
a fixed channel permutation applied to both queries and keys.

Decode with pre-rotation keys: the cache holds keys as they were before the
rotation (quantized ones and the fp16 window alike); token t of the sequence
sits at position t (quantized tokens first, then the window, as in the
cache), and the query arrives already rotated to its own position.  The
score of token t is ``alpha * q . rope(Khat[t], t)``, in fp64.
"""

import numpy as np

from .attention import attention
from .cache import context


def thetas(head_dim, base):
    """fp64 [D/2]: theta_f = base^(-2f/D)."""
    f = np.arange(head_dim // 2, dtype=np.float64)
    return np.float64(base) ** (-2.0 * f / head_dim)


def rope(x, positions, base):
    """Rotate rows of x (fp64 [T, D]) by their positions (int [T]); fp64."""
    x = np.asarray(x, dtype=np.float64)
    T, D = x.shape
    ang = np.asarray(positions, dtype=np.float64)[:, None] * thetas(D, base)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[:, 0::2], x[:, 1::2]
    y = np.empty_like(x)
    y[:, 0::2] = a * c - b * s
    y[:, 1::2] = a * s + b * c
    return y


def decode_head_rope(q, state, alpha, group, bits, base):
    """Decode output (fp64 [D]) of one (sequence, head) cache state whose
    keys are stored before the rotation; q is the rotated query."""
    kk, vv = context(state, group, bits)
    return attention(q, rope(kk, np.arange(kk.shape[0]), base), vv, alpha)
