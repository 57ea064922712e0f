"""Every compiled code width and group size, B in {2, 4, 8} x G in {32, 64,
128}, on a small ragged batch through the C ABI against the oracle: the
prefilled cache bit for bit, the plain, the pre-rotation-key and the
attention-sink (5 fp16 sink tokens, with and without the rotation) decode
within
max-abs 2e-3 / relative L2 1e-3 of the fp64 oracle, and a flush of the full
windows bit for bit.  Batch 9 x 32 heads (288 pairs) runs the decode with one
sub-chunk in flight per wave (more workgroups than compute units), batch 2
with two (and several workgroups per pair where the context is long)."""

import numpy as np
import pytest
import torch

from bit_kv_cache_decode_amd import kivi
from oracle import cache as ocache
from oracle import rope as orope
from oracle import sink as osink
from tests.gpu_common import assert_head_bit_exact, assert_within_tolerance, head_buffers

pytestmark = pytest.mark.gpu

D, H, R, CAP = 128, 32, 128, 640


def _case(bits, G, batch, seed):
    rng = np.random.default_rng(seed)
    T = CAP
    k = rng.standard_normal((batch, H, T, D), np.float32)
    k[:, :, :, 5] *= 40.0                                # an outlier key channel
    k = k.astype(np.float16)
    v = rng.standard_normal((batch, H, T, D), np.float32).astype(np.float16)
    q = (rng.standard_normal((batch, H, D), np.float32) / np.sqrt(D)).astype(np.float16)
    base = [0, 1, G - 1, G, G + 5, 2 * G + R - 1, R, 3 * G + 17, 500]
    lens = np.array([base[i % len(base)] for i in range(batch)], np.int32)
    win = np.array([n % G for n in lens], np.int32)
    if batch > 1:
        win[1] = min(int(lens[1]), R)                    # a window-only sequence
        win[-1] = R                                      # a full window (flushed below)
        lens[-1] = 2 * G + R
    return k, v, q, lens, win


@pytest.mark.parametrize("batch", [2, 9])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_width_group_combination(bits, G, batch):
    seed = 3000 + 10 * bits + G + batch
    k, v, q, lens, win = _case(bits, G, batch, seed)
    c = kivi.KiviCache(batch, H, D, bits, G, R, CAP)
    kivi.prefill(c, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                 torch.from_numpy(lens).cuda(), torch.from_numpy(win).cuda())
    qt = torch.from_numpy(q).cuda()
    out = kivi.decode_attn(c, qt, 1.0).cpu().numpy()
    out_r = kivi.decode_attn_rope(c, qt, 1.0, 10000.0).cpu().numpy()
    srng = np.random.default_rng(seed + 1)
    sk = (srng.standard_normal((batch, H, 5, D), np.float32) * 3).astype(np.float16)
    sv = srng.standard_normal((batch, H, 5, D), np.float32).astype(np.float16)
    skt, svt = torch.from_numpy(sk).cuda(), torch.from_numpy(sv).cuda()
    out_s = kivi.decode_attn_sink(c, qt, 1.0, skt, svt).cpu().numpy()
    out_rs = kivi.decode_attn_sink(c, qt, 1.0, skt, svt, rope_base=10000.0).cpu().numpy()
    assert c.status_bits() == 0
    heads = [(b, h) for b in range(batch) for h in (0, 13, 31)]
    for b, h in heads:
        st = ocache.head_state(k[b, h], v[b, h], int(lens[b] - win[b]), int(win[b]), G, bits,
                               CAP, R)
        if h == 0:
            assert_head_bit_exact(head_buffers(c, b, h), st, G)
        ref = ocache.decode_head(q[b, h], st, 1.0, G, bits)
        assert_within_tolerance(out[b, h], ref, f"plain b={b} h={h}")
        ref_r = orope.decode_head_rope(q[b, h], st, 1.0, G, bits, 10000.0)
        assert_within_tolerance(out_r[b, h], ref_r, f"rope b={b} h={h}")
        ref_s = osink.decode_head_sink(q[b, h], st, sk[b, h], sv[b, h], 1.0, G, bits)
        assert_within_tolerance(out_s[b, h], ref_s, f"sink b={b} h={h}")
        ref_rs = osink.decode_head_sink(q[b, h], st, sk[b, h], sv[b, h], 1.0, G, bits,
                                        rope_base=10000.0)
        assert_within_tolerance(out_rs[b, h], ref_rs, f"rotary sink b={b} h={h}")
    # flush: only the full window moves, bit for bit as the oracle encodes it
    kivi.flush_residual(c)
    torch.cuda.synchronize()
    ql = c.q_len.cpu().numpy()
    rl = c.r_len.cpu().numpy()
    full = win == R
    assert np.array_equal(ql, np.where(full, lens, lens - win))
    assert np.array_equal(rl, np.where(full, 0, win))
    for b in np.flatnonzero(full):
        for h in (0, 31):
            t0 = int(lens[b] - R)
            enc = ocache.encode_tokens(k[b, h, t0:t0 + R], v[b, h, t0:t0 + R], G, bits)
            for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
                got = getattr(c, name)[b, h, t0 // G:(t0 + R) // G].cpu().numpy()
                assert np.array_equal(got.view(np.uint8), enc[name].view(np.uint8)), (name, b, h)
    assert not c.tickets.any() and c.status_bits() == 0



@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("bits", [2, 4])
def test_two_word_lanes_width_group(bits, G):
    """The decode that holds two code words per lane, selected by capacity
    (8 x 32 pairs, one workgroup each, and at least 16 sub-chunks per wave in
    a cache of 16384 tokens), for every width and group it is built for.  The
    sequences are short and ragged: empty, window only, one tile plus one
    window token, 1024 + G quantized tokens (at B=2 and G=32 the last
    sub-chunk holds one valid tile), full windows and partial ones.  Sampled
    heads against the oracle."""
    batch, cap = 8, 16384
    ql = np.array([0, 0, G, 1024 + G, 2048, 768, G, 2048 - G], np.int32)
    win = np.array([0, 1, 1, R, R, 9, G, 52], np.int32)
    lens = ql + win
    rng = np.random.default_rng(5000 + 10 * bits + G)
    T = int(lens.max())
    k = rng.standard_normal((batch, H, T, D), np.float32)
    k[:, :, :, 5] *= 40.0
    k = k.astype(np.float16)
    v = rng.standard_normal((batch, H, T, D), np.float32).astype(np.float16)
    q = (rng.standard_normal((batch, H, D), np.float32) / np.sqrt(D)).astype(np.float16)
    c = kivi.KiviCache(batch, H, D, bits, G, R, cap)
    assert kivi.decode_splits(c.dims) == 1
    kivi.prefill(c, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                 torch.from_numpy(lens).cuda(), torch.from_numpy(win).cuda())
    out = kivi.decode_attn(c, torch.from_numpy(q).cuda(), 1.0).cpu().numpy()
    assert c.status_bits() == 0
    for b in range(batch):
        for h in (0, 13, 31):
            st = ocache.head_state(k[b, h], v[b, h], int(ql[b]), int(win[b]), G, bits, cap, R)
            ref = ocache.decode_head(q[b, h], st, 1.0, G, bits)
            assert_within_tolerance(out[b, h], ref, f"b={b} h={h} q_len={ql[b]} win={win[b]}")
