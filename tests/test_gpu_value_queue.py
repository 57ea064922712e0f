"""GPU parity of the value-queue cache (discosf KIVI tutorial, section 3.2:
values leave an fp16 queue of the newest R one token at a time, quantized per
token as they leave; keys flushed R at a time) against ``oracle.value_queue``,
through the C ABI: kivi_prefill_vq, kivi_append_kv_vq, kivi_flush_residual_vq
and kivi_decode_attn_vq.

Buffers (codes, zero-points, steps, key window, value ring, lengths) must
match the oracle bit for bit; decode outputs must be within max-abs 2e-3 and
relative L2 1e-3 of the oracle's fp64 attention over the same context."""

import numpy as np
import pytest
import torch

from bit_kv_cache_decode_amd import kivi
from oracle import value_queue as ovq
from tests.gpu_common import assert_within_tolerance, parallel_map, workload

pytestmark = pytest.mark.gpu


def _gpu_vq(w, n, r, dims=None):
    """Value-queue cache on the GPU holding tokens [0, n) of workload w, r of
    them in the key window (per sequence)."""
    d = dict(w.dims()) if dims is None else dims
    c = kivi.KiviCache(**d)
    kivi.prefill_vq(c, torch.from_numpy(w.k).cuda(), torch.from_numpy(w.v).cuda(),
                    torch.from_numpy(np.asarray(n, np.int32)).cuda(),
                    torch.from_numpy(np.asarray(r, np.int32)).cuda())
    torch.cuda.synchronize()
    return c


def _oracle_vq(w, n, r, dims=None):
    d = dict(w.dims()) if dims is None else dims
    o = ovq.ValueQueueCache(d["batch"], d["heads"], d["head_dim"], d["bits"], d["group"],
                            d["residual"], d["capacity"])
    o.prefill(w.k[:d["batch"]], w.v[:d["batch"]], np.asarray(n), np.asarray(r))
    return o


def _assert_same_buffers(c, o):
    assert np.array_equal(c.q_len.cpu().numpy(), o.q_len)
    assert np.array_equal(c.r_len.cpu().numpy(), o.r_len)
    assert c.status_bits() == 0 and o.status == 0
    for name in ("k_codes", "v_codes", "k_zero", "k_scale", "v_zero", "v_scale", "v_res"):
        got = getattr(c, name).cpu().numpy()
        assert np.array_equal(got.view(np.uint8), getattr(o, name).view(np.uint8)), name
    kr = c.k_res.cpu().numpy()
    for b in range(o.batch):     # the key window's live rows
        r = int(o.r_len[b])
        assert np.array_equal(kr[b, :, :r].view(np.uint16), o.k_res[b, :, :r].view(np.uint16))


def _check_decode(c, o, q, alpha, heads=None):
    out = kivi.decode_attn_vq(c, torch.from_numpy(q).cuda(), alpha)
    torch.cuda.synchronize()
    assert c.status_bits() == 0
    out = out.cpu().numpy()
    heads = heads or [(b, h) for b in range(o.batch) for h in range(o.heads)]

    def one(bh):
        b, h = bh
        ref = ovq.decode_head(q[b, h], o.head(b, h), alpha, o.G, o.bits, o.R)
        return assert_within_tolerance(out[b, h], ref, f"b={b} h={h}")
    return parallel_map(one, heads)


@pytest.mark.parametrize("number,batch", [(1, None), (2, 2), (3, 2)])
def test_prefill_and_decode_match_oracle(number, batch):
    """The tiny, 7B and 13B layer shapes (all heads of the sequences kept):
    the prefilled buffers bit for bit, every head's decode to tolerance."""
    w = workload(number, batch=batch)
    n, r = w.lengths, w.r_len
    c, o = _gpu_vq(w, n, r), _oracle_vq(w, n, r)
    _assert_same_buffers(c, o)
    _check_decode(c, o, w.q, w.config.sm_scale)


@pytest.mark.parametrize("n,r", [(0, 0), (5, 5), (31, 31), (32, 0), (33, 1), (64, 0), (100, 4),
                                 (255, 31), (256, 0)])
def test_edge_lengths(n, r):
    """Empty; a queue that has not overflowed (T < R, T = R); the first
    evictions; a partly filled value tile; the capacity filled."""
    w = workload(1)
    c, o = _gpu_vq(w, [n], [r]), _oracle_vq(w, [n], [r])
    _assert_same_buffers(c, o)
    out = kivi.decode_attn_vq(c, torch.from_numpy(w.q).cuda(), w.config.sm_scale)
    torch.cuda.synchronize()
    if n == 0:
        assert not out.any()
    else:
        ref = ovq.decode_head(w.q[0, 0], o.head(0, 0), w.config.sm_scale, 32, 2, 32)
        assert_within_tolerance(out.cpu().numpy()[0, 0], ref, f"{n}/{r}")


@pytest.mark.parametrize("bits,G,R", [(2, 32, 128), (4, 32, 64), (8, 64, 128), (2, 128, 128),
                                      (4, 128, 256)])
def test_streaming_appends_and_key_flushes_match_oracle(bits, G, R):
    """Token-by-token appends (each followed by a key flush) from a prefilled
    start, on the GPU and in the oracle: the buffers bit for bit after every
    few steps and the decode at the end, across evictions and key flushes."""
    rng = np.random.default_rng(1000 + bits + G + R)
    B, H, D = 2, 3, 128
    n0 = np.array([2 * G + 5, R + G], np.int32)
    steps = R + G + 7
    cap = ((int(n0.max()) + steps) // G + 2) * G
    T = int(n0.max()) + steps
    k = rng.standard_normal((B, H, T, D), np.float32)
    k[..., 11] *= 25.0
    k = k.astype(np.float16)
    v = rng.standard_normal((B, H, T, D), np.float32).astype(np.float16)
    r0 = n0 % G
    c = kivi.KiviCache(B, H, D, bits, G, R, cap)
    kivi.prefill_vq(c, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                    torch.from_numpy(n0).cuda(), torch.from_numpy(r0.astype(np.int32)).cuda())
    o = ovq.ValueQueueCache(B, H, D, bits, G, R, cap)
    o.prefill(k, v, n0, r0)
    kt, vt = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    b_idx = np.arange(B)
    for s in range(steps):
        t = n0 + s
        kn = np.ascontiguousarray(k[b_idx, :, t])
        vn = np.ascontiguousarray(v[b_idx, :, t])
        kivi.append_kv_vq(c, torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda())
        kivi.flush_residual_vq(c)
        o.append(kn, vn)
        o.flush()
        if s % 37 == 0 or s == steps - 1:
            torch.cuda.synchronize()
            _assert_same_buffers(c, o)
    del kt, vt
    q = (rng.standard_normal((B, H, D)) / np.sqrt(D)).astype(np.float16)
    _check_decode(c, o, q, 1.0)


def test_ragged_batch_and_split_decode():
    """Eight sequences of the ragged workload (every split of quantized keys,
    quantized values and fp16 values), then the same contents at a capacity
    that splits each (sequence, head) over several workgroups."""
    w = workload(4, batch=8)
    n, r = w.lengths, w.r_len
    c, o = _gpu_vq(w, n, r), _oracle_vq(w, n, r)
    _assert_same_buffers(c, o)
    rng = np.random.default_rng(44)
    heads = sorted({(int(b), int(h)) for b, h in zip(rng.integers(0, 8, 40), rng.integers(0, 32, 40))})
    _check_decode(c, o, w.q, 1.0, heads)
    w2 = workload(2, batch=2)
    d = dict(w2.dims(), capacity=65536)
    c2, o2 = _gpu_vq(w2, w2.lengths, w2.r_len, d), _oracle_vq(w2, w2.lengths, w2.r_len, d)
    assert kivi.decode_splits(c2.dims) > 1
    _check_decode(c2, o2, w2.q, 1.0, [(0, 0), (1, 13), (1, 31)])


def test_queue_differs_from_window_flush_only_in_the_values():
    """The same tokens in a value-queue cache and a window-flush cache: the
    keys are bit-identical, the decodes differ (the queue keeps the newest R
    values in fp16)."""
    w = workload(2, batch=1)
    c = _gpu_vq(w, w.lengths, w.r_len)
    from tests.gpu_common import gpu_cache
    p = gpu_cache(w)
    for name in ("k_codes", "k_zero", "k_scale", "q_len", "r_len"):
        assert torch.equal(getattr(c, name), getattr(p, name)), name
    q = torch.from_numpy(w.q).cuda()
    a = kivi.decode_attn_vq(c, q, 1.0)
    b = kivi.decode_attn(p, q, 1.0)
    torch.cuda.synchronize()
    # w has a full 128-token window: the queue holds the same 128 values in
    # fp16 that the window-flush cache holds, so both attend over the same
    # values here; one more token makes them differ (up to rounding: the
    # plain decode sums in another lane order than the value-queue decode)
    assert torch.allclose(a, b, rtol=1e-4, atol=1e-4)
    kn = torch.from_numpy(w.k[:, :, 0]).cuda().contiguous()
    kivi.append_kv_vq(c, kn, kn)    # the window is full: refused
    torch.cuda.synchronize()
    assert c.status_bits() == kivi.ST_RESIDUAL_FULL
