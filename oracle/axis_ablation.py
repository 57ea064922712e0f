"""Axis ablation of the quantized KV cache (oracle-side analysis).

Test and analysis infrastructure only (see ``oracle/__init__.py``): it uses
the oracle's quantizer and attention and nothing from the product path.

The unite.ai axis-selection guide argues the choice of grouping axis from the
error model (quantization-error section: a group's step is its range over the
levels, so one large member coarsens every other member of its group), the
key statistics (keys section: a few channels carry large magnitudes on every
token, so keys are grouped per channel) and the value statistics (values
section: values have no such channels and enter the output as a weighted sum
over tokens, so they are grouped per token).  The discosf KIVI tutorial
(section 2.2) states the same asymmetric choice.

This module quantizes the same keys and values with each of the four axis
choices -- keys per channel (G tokens of one channel) or per token (G
channels of one token), values likewise -- with the one quantizer, and
measures on the exact dequantization:

* key error, two ways: mean |K_hat - K| / mean |K| (every entry counts
  alike) and ||K_hat - K||_F / ||K||_F (dominated by the large channels);
* score error: ||(K_hat - K) q||_2 / ||K q||_2 (scores before the softmax
  scale, which cancels);
* output error: ||o(K_hat, V_hat) - o(K, V)||_2 / ||o(K, V)||_2 with o the
  fp64 attention of one query over all tokens.

Direction only: the guide's own figures come from real model activations;
here the keys and values are the seeded synthetic workloads (outlier key
channels as in the guide's keys section).

``python -m tests.test_axis_ablation`` prints the table for the
Llama-2-7B-shaped workload (a few seconds).
"""

import numpy as np

from .attention import attention
from .quantizer import (dequantize_keys, dequantize_values, quantize_keys,
                        quantize_values)

AXES = ("channel", "token")


def quantize_axis(x, axis, group, bits):
    """Exact fp64 dequantization of fp16 ``x`` [L, D] quantized in groups of
    ``group`` tokens of one channel (axis "channel") or ``group`` channels of
    one token (axis "token")."""
    if axis == "channel":
        return dequantize_keys(*quantize_keys(x, group, bits), group)
    if axis == "token":
        return dequantize_values(*quantize_values(x, group, bits), group)
    raise ValueError("axis must be 'channel' or 'token'")


def errors(k, v, q, alpha, group, bits, k_axis, v_axis):
    """The relative errors of one (sequence, head) for one axis choice."""
    kf = k.astype(np.float64)
    vf = v.astype(np.float64)
    qf = np.asarray(q, dtype=np.float64)
    kh = quantize_axis(k, k_axis, group, bits)
    vh = quantize_axis(v, v_axis, group, bits)
    ref = attention(qf, kf, vf, alpha)
    return {
        "key_mean": float(np.abs(kh - kf).mean() / np.abs(kf).mean()),
        "key": float(np.linalg.norm(kh - kf) / np.linalg.norm(kf)),
        "score": float(np.linalg.norm((kh - kf) @ qf) / np.linalg.norm(kf @ qf)),
        "output": float(np.linalg.norm(attention(qf, kh, vh, alpha) - ref) / np.linalg.norm(ref)),
    }


def ablate(heads, alpha, group, bits):
    """Mean of each error over ``heads`` (a list of (k, v, q)) for every
    (key axis, value axis) pair."""
    out = {}
    for ka in AXES:
        for va in AXES:
            per = [errors(k, v, q, alpha, group, bits, ka, va) for k, v, q in heads]
            out[(ka, va)] = {m: float(np.mean([p[m] for p in per]))
                             for m in ("key_mean", "key", "score", "output")}
    return out


def table(results):
    lines = ["| keys grouped per | values grouped per | key error (mean abs) | key error (Frobenius) "
             "| score error | output error |",
             "|---|---|---:|---:|---:|---:|"]
    for (ka, va), r in results.items():
        lines.append(f"| {ka} | {va} | {r['key_mean']:.4f} | {r['key']:.4f} | {r['score']:.4f} "
                     f"| {r['output']:.4f} |")
    return "\n".join(lines)
