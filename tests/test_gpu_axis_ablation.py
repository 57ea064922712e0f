"""The axis ablation on GPU-encoded caches.  The library's encoder groups
its first operand per channel (G tokens of one channel, the key axis) and
its second per token (G channels of one token, the value axis), so a
prefill with keys and values swapped is the flipped-axis encoder: keys per
token, values per channel.  Its dequantized buffers must equal the oracle's
flipped-axis quantization bit for bit, so every ablation error measured on
GPU-encoded caches is the oracle's own (the direction itself is pinned on
the CPU)."""

import numpy as np
import pytest
import torch

from bit_kv_cache_decode_amd import kivi
from oracle import axis_ablation as oab
from oracle import cache as ocache
from tests.gpu_common import head_buffers, workload

pytestmark = pytest.mark.gpu


def _encode(w, first, second):
    """All 4096 tokens of every head quantized (no window); the first
    operand takes the key grouping, the second the value grouping."""
    d = w.dims()
    c = kivi.KiviCache(**d)
    n = torch.full((w.q.shape[0],), w.config.context, dtype=torch.int32, device="cuda")
    kivi.prefill(c, torch.from_numpy(first).cuda(), torch.from_numpy(second).cuda(), n,
                 torch.zeros_like(n))
    torch.cuda.synchronize()
    assert c.status_bits() == 0
    return c


@pytest.mark.parametrize("bits", [2, 4])
def test_flipped_axis_encoding_matches_the_oracle(bits):
    w = workload(2, bits=bits, batch=1)
    G = w.config.group
    normal = _encode(w, w.k, w.v)
    flipped = _encode(w, w.v, w.k)
    for h in (0, 11, 31):
        k, v = w.k[0, h], w.v[0, h]
        kc, vt = ocache.context(head_buffers(normal, 0, h), G, bits)     # K per channel, V per token
        vc, kt = ocache.context(head_buffers(flipped, 0, h), G, bits)    # V per channel, K per token
        assert np.array_equal(kc, oab.quantize_axis(k, "channel", G, bits))
        assert np.array_equal(vt, oab.quantize_axis(v, "token", G, bits))
        assert np.array_equal(kt, oab.quantize_axis(k, "token", G, bits))
        assert np.array_equal(vc, oab.quantize_axis(v, "channel", G, bits))
