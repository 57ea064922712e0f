"""GPU parity of kivi_decode_attn_rope (keys stored before the rotary
embedding, rotated by their positions after dequantization; the guide's
rotary-embedding section) against the oracle's fp64 decode, to the same
tolerance as the plain decode (max-abs 2e-3, relative L2 1e-3).  The
workloads' queries stand for already rotated ones."""

import numpy as np
import pytest
import torch

from bit_kv_cache_decode_amd import kivi
from oracle import cache as ocache
from oracle import rope as orope
from tests.gpu_common import assert_within_tolerance, gpu_cache, oracle_head, workload

pytestmark = pytest.mark.gpu


def _rope_heads(c, w, heads, base=10000.0):
    q = torch.from_numpy(w.q).cuda()
    out = kivi.decode_attn_rope(c, q, w.config.sm_scale, base)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    G = w.config.group
    worst = 0.0
    for b, h in heads:
        st = oracle_head(w, b, h)
        ref = orope.decode_head_rope(w.q[b, h], st, w.config.sm_scale, G, w.bits, base)
        mx, _ = assert_within_tolerance(out[b, h], ref, f"b={b} h={h}")
        worst = max(worst, mx)
        # the rotation matters for these heads: the plain decode differs
    assert c.status_bits() == 0
    return out, worst


def test_rope_llama2_7b_shape_all_heads():
    w = workload(2, batch=2)
    c = gpu_cache(w)
    out, _ = _rope_heads(c, w, [(b, h) for b in range(2) for h in range(32)])
    plain = kivi.decode_attn(c, torch.from_numpy(w.q).cuda(), 1.0).cpu().numpy()
    assert np.abs(out - plain).max() > 1e-2   # the keys were rotated


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_rope_long_context_sampled_heads(bits):
    """Positions up to 131071: the angles' fp64 revolutions keep the
    rotation exact enough at every position."""
    w = workload(5, bits=bits)
    c = gpu_cache(w)
    _rope_heads(c, w, [(0, 0), (0, 13), (0, 31)])


@pytest.mark.parametrize("bits", [4, 8])
def test_rope_13b_shape_sampled_heads(bits):
    """640 (sequence, head) pairs (more workgroups than compute units)."""
    w = workload(3, bits=bits)
    c = gpu_cache(w)
    _rope_heads(c, w, [(0, 0), (7, 21), (15, 39)])


@pytest.mark.parametrize("q_len,r_len", [(0, 1), (0, 128), (32, 0), (3968, 0), (4064, 31)])
def test_rope_edge_lengths(q_len, r_len):
    w = workload(2, batch=1)
    c = gpu_cache(w, q_len=[q_len], r_len=[r_len])
    q = torch.from_numpy(w.q).cuda()
    out = kivi.decode_attn_rope(c, q, 1.0, 10000.0).cpu().numpy()
    for h in (0, 31):
        st = ocache.head_state(w.k[0, h], w.v[0, h], q_len, r_len, 32, 2, 4096, 128)
        ref = orope.decode_head_rope(w.q[0, h], st, 1.0, 32, 2, 10000.0)
        assert_within_tolerance(out[0, h], ref, f"{q_len}+{r_len}")


@pytest.mark.parametrize("base", [500.0, 500000.0])
def test_rope_other_bases_and_splits(base):
    """Other rotary bases, and a capacity that splits each (sequence, head)
    over several workgroups (the split merge with rotated keys)."""
    w = workload(2, batch=2)
    c = gpu_cache(w, capacity=65536)
    assert kivi.decode_splits(c.dims) > 1
    q = torch.from_numpy(w.q).cuda()
    out = kivi.decode_attn_rope(c, q, 1.0, base).cpu().numpy()
    for b, h in [(0, 0), (1, 17), (1, 31)]:
        st = oracle_head(w, b, h, capacity=65536)
        ref = orope.decode_head_rope(w.q[b, h], st, 1.0, 32, 2, base)
        assert_within_tolerance(out[b, h], ref, f"base {base}")
