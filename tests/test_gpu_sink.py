"""GPU parity of kivi_decode_attn_sink (an fp16 attention-sink segment
ahead of the cache's tokens; the guide's future-directions section) against
the oracle's fp64 decode, to the plain decode's tolerance (max-abs 2e-3,
relative L2 1e-3).  Sink rows come from the seeded sink generator: sink
token 0 draws a large score, the rest are N(0, 9) keys and N(0, 1) values."""

import numpy as np
import pytest
import torch

from bit_kv_cache_decode_amd import kivi
from bit_kv_cache_decode_amd import workloads as wl
from oracle import cache as ocache
from oracle import sink as osink
from tests.gpu_common import assert_within_tolerance, gpu_cache, oracle_head, workload

pytestmark = pytest.mark.gpu


def _run(c, w, n_sink, rope_base=0.0):
    ks, vs = wl.sink_tokens(w, n_sink)
    q = torch.from_numpy(w.q).cuda()
    out = kivi.decode_attn_sink(c, q, w.config.sm_scale, torch.from_numpy(ks).cuda(),
                                torch.from_numpy(vs).cuda(), rope_base=rope_base)
    torch.cuda.synchronize()
    assert c.status_bits() == 0
    return out.cpu().numpy(), ks, vs


def _check(out, w, ks, vs, heads, state=oracle_head, rope_base=None):
    G = w.config.group
    for b, h in heads:
        st = state(w, b, h)
        ref = osink.decode_head_sink(w.q[b, h], st, ks[b, h], vs[b, h], w.config.sm_scale, G,
                                     w.bits, rope_base=rope_base)
        assert_within_tolerance(out[b, h], ref, f"b={b} h={h}")


@pytest.mark.parametrize("n_sink", [4, 64])
def test_sink_llama2_7b_shape_all_heads(n_sink):
    w = workload(2, batch=2)
    c = gpu_cache(w)
    out, ks, vs = _run(c, w, n_sink)
    _check(out, w, ks, vs, [(b, h) for b in range(2) for h in range(32)])
    plain = kivi.decode_attn(c, torch.from_numpy(w.q).cuda(), 1.0).cpu().numpy()
    assert np.abs(out - plain).max() > 1e-2   # the sink took part


def test_no_sink_is_bit_identical_to_decode_attn():
    w = workload(2, batch=2)
    c = gpu_cache(w)
    out, _, _ = _run(c, w, 0)
    plain = kivi.decode_attn(c, torch.from_numpy(w.q).cuda(), 1.0).cpu().numpy()
    assert np.array_equal(out, plain)


@pytest.mark.parametrize("q_len,r_len,n_sink", [(0, 0, 1), (0, 0, 33), (0, 5, 7), (32, 0, 8),
                                                (4064, 31, 4096), (3968, 128, 2)])
def test_sink_edge_lengths(q_len, r_len, n_sink):
    """Empty caches (the sink alone), one sink token, shares that leave most
    waves without sink tokens, and the largest sink (512 tokens a wave)."""
    w = workload(2, batch=1)
    c = gpu_cache(w, q_len=[q_len], r_len=[r_len])
    out, ks, vs = _run(c, w, n_sink)

    def state(w, b, h):
        return ocache.head_state(w.k[b, h], w.v[b, h], q_len, r_len, 32, 2, 4096, 128)
    _check(out, w, ks, vs, [(0, 0), (0, 17), (0, 31)], state)


def test_sink_with_splits():
    """A capacity that splits each (sequence, head) over several workgroups:
    the sink is shared over every split's waves and merged with the rest."""
    w = workload(2, batch=2)
    c = gpu_cache(w, capacity=65536)
    assert kivi.decode_splits(c.dims) > 1
    out, ks, vs = _run(c, w, 100)
    _check(out, w, ks, vs, [(0, 0), (1, 9), (1, 31)])


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_sink_13b_shape_sampled_heads(bits):
    """640 (sequence, head) pairs: the kernels of grids above one workgroup
    per compute unit."""
    w = workload(3, bits=bits)
    c = gpu_cache(w)
    out, ks, vs = _run(c, w, 16)
    _check(out, w, ks, vs, [(0, 0), (7, 21), (15, 39)])


@pytest.mark.parametrize("bits", [2, 4])
def test_sink_long_context_sampled_heads(bits):
    w = workload(5, bits=bits)
    c = gpu_cache(w)
    out, ks, vs = _run(c, w, 4)
    _check(out, w, ks, vs, [(0, 0), (0, 31)])


# ---- keys (the sink's too) stored before the rotary embedding: sink token s
# at position s, the cache's tokens after the sink

def test_rotary_sink_llama2_7b_shape_all_heads():
    w = workload(2, batch=2)
    c = gpu_cache(w)
    out, ks, vs = _run(c, w, 4, rope_base=10000.0)
    _check(out, w, ks, vs, [(b, h) for b in range(2) for h in range(32)], rope_base=10000.0)


def test_rotary_no_sink_is_bit_identical_to_decode_attn_rope():
    w = workload(2, batch=2)
    c = gpu_cache(w)
    out, _, _ = _run(c, w, 0, rope_base=10000.0)
    ref = kivi.decode_attn_rope(c, torch.from_numpy(w.q).cuda(), 1.0, 10000.0).cpu().numpy()
    assert np.array_equal(out, ref)


@pytest.mark.parametrize("q_len,r_len,n_sink", [(0, 0, 9), (0, 5, 7), (32, 0, 8), (4064, 31, 100)])
def test_rotary_sink_edge_lengths(q_len, r_len, n_sink):
    w = workload(2, batch=1)
    c = gpu_cache(w, q_len=[q_len], r_len=[r_len])
    out, ks, vs = _run(c, w, n_sink, rope_base=10000.0)

    def state(w, b, h):
        return ocache.head_state(w.k[b, h], w.v[b, h], q_len, r_len, 32, 2, 4096, 128)
    _check(out, w, ks, vs, [(0, 0), (0, 31)], state, rope_base=10000.0)


@pytest.mark.parametrize("workload_number,bits", [(3, 4), (5, 4)])
def test_rotary_sink_large_grids_and_long_context(workload_number, bits):
    """The depth-1 rotary kernel (13B shape at B=4) and split merges with
    positions up to 131075 (131072-token workload)."""
    w = workload(workload_number, bits=bits)
    c = gpu_cache(w)
    out, ks, vs = _run(c, w, 4, rope_base=10000.0)
    heads = [(0, 0), (7, 21), (15, 39)] if workload_number == 3 else [(0, 0), (0, 31)]
    _check(out, w, ks, vs, heads, rope_base=10000.0)


# ---- the whole step with a sink: one kernel where a workgroup covers a
# (sequence, head), else the three calls

@pytest.mark.parametrize("batch,case", [(8, "fills"), (2, "fills"), (8, "append_only"),
                                        (8, "long_window")])
def test_step_with_sink_matches_three_calls_and_oracle(batch, case):
    """The step with a sink in one kernel (batch 8) or three (batch 2), for a
    step whose append fills the window (flushed from registers), an append
    that leaves it short of full (the common step), and a 256-token window
    (flushed by re-reading it through LDS): the cache as the three calls
    leave it, bit for bit, and the output against the oracle."""
    w = workload(2, batch=batch) if batch != 8 else workload(2)
    B = w.q.shape[0]
    R = 256 if case == "long_window" else 128
    ql = w.q_len - (128 if case == "long_window" else 0)
    rl = {"fills": w.r_len - 1, "append_only": w.r_len - 3,
          "long_window": np.full(B, 255, np.int32)}[case].astype(np.int32)
    base = gpu_cache(w, q_len=ql, r_len=rl, residual=R)
    assert kivi.decode_step_kernels(base.dims) == (1 if batch == 8 else 3)
    last = ql + rl                                           # the appended token
    k_new = torch.from_numpy(np.ascontiguousarray(w.k[np.arange(B), :, last])).cuda()
    v_new = torch.from_numpy(np.ascontiguousarray(w.v[np.arange(B), :, last])).cuda()
    ks, vs = wl.sink_tokens(w, 8)
    kst, vst = torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda()
    q = torch.from_numpy(w.q).cuda()
    a = kivi.KiviCache(**base.shape)
    b = kivi.KiviCache(**base.shape)
    for c in (a, b):
        for n, t in base.buffers().items():
            getattr(c, n).copy_(t)
    out_a = kivi.decode_step_sink(a, k_new, v_new, q, 1.0, kst, vst)
    kivi.append_kv(b, k_new, v_new)
    out_b = kivi.decode_attn_sink(b, q, 1.0, kst, vst)
    kivi.flush_residual(b)
    torch.cuda.synchronize()
    for n, t in a.buffers().items():
        assert torch.equal(t, getattr(b, n)), n
    flushed = case != "append_only"
    assert a.r_len.cpu().tolist() == ([0] * B if flushed else (rl + 1).tolist())
    assert a.status_bits() == 0
    assert torch.allclose(out_a, out_b, rtol=1e-5, atol=1e-6)
    out = out_a.cpu().numpy()

    # the oracle over the state before any flush (every token in place)
    def state(w, bb, h):
        return ocache.head_state(w.k[bb, h], w.v[bb, h], int(ql[bb]), int(rl[bb]) + 1, 32, 2,
                                 4096, R)
    _check(out, w, ks, vs, [(0, 0), (B - 1, 31), (B // 2, 7)], state)


def test_step_with_no_sink_is_the_plain_step():
    w = workload(2)
    base = gpu_cache(w, q_len=w.q_len, r_len=w.r_len - 1)
    B = w.q.shape[0]
    last = w.lengths - 1
    k_new = torch.from_numpy(np.ascontiguousarray(w.k[np.arange(B), :, last])).cuda()
    v_new = torch.from_numpy(np.ascontiguousarray(w.v[np.arange(B), :, last])).cuda()
    empty = torch.empty((B, 32, 0, 128), dtype=torch.float16, device="cuda")
    q = torch.from_numpy(w.q).cuda()
    a = kivi.KiviCache(**w.dims())
    b = kivi.KiviCache(**w.dims())
    for c in (a, b):
        for n, t in base.buffers().items():
            getattr(c, n).copy_(t)
    out_a = kivi.decode_step_sink(a, k_new, v_new, q, 1.0, empty, empty)
    out_b = kivi.decode_step(b, k_new, v_new, q, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    for n, t in a.buffers().items():
        assert torch.equal(t, getattr(b, n)), n
