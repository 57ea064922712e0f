"""Uniform asymmetric B-bit quantizer and the two grouping axes (oracle).

Test infrastructure only (see ``oracle/__init__.py``).

Definition followed (unite.ai axis-selection guide, section on what
quantization error is made of): the group minimum is the zero-point; the step
is the group's range divided by the number of representable levels minus one,
2^B - 1; every element is rounded to the nearest step.  Consequences the tests
pin: each element's error is at most half a step, and one outlier inflates the
step of its whole group.

Axes (same guide, keys and values sections; discosf KIVI tutorial sections 2.1
and 3.1): keys are grouped per channel over G consecutive tokens, values per
token over G consecutive channels.

The exact fp32 operation sequence (one IEEE rounding per operation, round to
nearest even, no fused multiply-add), which the GPU encoder must reproduce
bit for bit:

1. ``mn = float32(min x) + 0.0``, ``mx = float32(max x) + 0.0`` (adding +0
   turns a -0 into +0, so neither the stored zero-point nor the step of an
   all-zero group depends on the order of signed zeros); both exact because
   x is fp16.
2. ``step32 = (mx - mn) / float32(2^B - 1)``.
3. ``scale = float16(step32)`` (round to nearest even); ``s = float32(scale)``.
4. ``code = 0`` if ``s == 0``, else
   ``clip(rint_half_even((x - mn) / s), 0, 2^B - 1)`` -- a true division by
   the stored step, not a multiplication by its reciprocal.
5. stored ``zero = float16(mn)`` (exact) and stored ``scale``.
"""

import numpy as np

F32 = np.float32


def quantize_groups(x, bits):
    """Quantize every row of ``x`` (fp16, shape [..., n]) as one group.

    Returns ``(codes uint8 [..., n], zero fp16 [...], scale fp16 [...])``.
    """
    x = np.asarray(x)
    if x.dtype != np.float16:
        raise TypeError("quantizer input must be float16")
    if bits not in (2, 4, 8):
        raise ValueError("bits must be 2, 4 or 8")
    xf = x.astype(F32)
    if not np.all(np.isfinite(xf)):
        raise ValueError("quantizer input must be finite")
    levels = F32(2 ** bits - 1)
    mn = (xf.min(axis=-1) + F32(0.0)).astype(F32)          # step 1
    mx = (xf.max(axis=-1) + F32(0.0)).astype(F32)
    step32 = ((mx - mn).astype(F32) / levels).astype(F32)   # step 2
    scale = step32.astype(np.float16)                       # step 3
    s = scale.astype(F32)
    nonzero = s != 0
    s_safe = np.where(nonzero, s, F32(1.0)).astype(F32)
    quotient = ((xf - mn[..., None]).astype(F32) / s_safe[..., None]).astype(F32)
    codes = np.clip(np.rint(quotient), F32(0.0), levels)    # step 4
    codes = np.where(nonzero[..., None], codes, F32(0.0))
    return codes.astype(np.uint8), mn.astype(np.float16), scale


def quantize_keys(k, group, bits):
    """Per-channel key quantization over groups of ``group`` tokens.

    k: fp16 [L, D] with L a multiple of ``group``.
    Returns codes uint8 [L, D], zero fp16 [L/G, D], scale fp16 [L/G, D].
    Group (g, d) is channel d of tokens [g*G, (g+1)*G).
    """
    L, D = k.shape
    if L % group:
        raise ValueError("key token count must be a multiple of the group size")
    tiles = k.reshape(L // group, group, D).transpose(0, 2, 1)   # [g, d, t]
    codes, zero, scale = quantize_groups(tiles, bits)
    return codes.transpose(0, 2, 1).reshape(L, D), zero, scale


def quantize_values(v, group, bits):
    """Per-token value quantization over groups of ``group`` channels.

    v: fp16 [L, D] with D a multiple of ``group``.
    Returns codes uint8 [L, D], zero fp16 [L, D/G], scale fp16 [L, D/G].
    Group (t, j) is channels [j*G, (j+1)*G) of token t.
    """
    L, D = v.shape
    if D % group:
        raise ValueError("head_dim must be a multiple of the group size")
    rows = v.reshape(L, D // group, group)
    codes, zero, scale = quantize_groups(rows, bits)
    return codes.reshape(L, D), zero, scale


def dequantize_keys(codes, zero, scale, group):
    """Exact fp64 reconstruction zero + code * scale for key groups."""
    z = np.repeat(zero.astype(np.float64), group, axis=0)
    s = np.repeat(scale.astype(np.float64), group, axis=0)
    return z + codes.astype(np.float64) * s


def dequantize_values(codes, zero, scale, group):
    """Exact fp64 reconstruction zero + code * scale for value groups."""
    z = np.repeat(zero.astype(np.float64), group, axis=1)
    s = np.repeat(scale.astype(np.float64), group, axis=1)
    return z + codes.astype(np.float64) * s
