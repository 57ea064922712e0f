"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Encoder outputs (codes, zero-points, steps, window rows, lengths) must match
the oracle bit for bit; decode outputs must be within max-abs 2e-3 and
relative L2 1e-3 of the oracle's fp64 attention on the same dequantized
values.  Workloads are the seeded synthetic ones of
``bit_kv_cache_decode_amd.workloads`` at their full sizes; where the oracle
would be slow, a fixed sample of (sequence, head) pairs is checked.
"""

import numpy as np
import pytest
import torch

from bit_kv_cache_decode_amd import kivi
from bit_kv_cache_decode_amd import workloads as wl
from oracle import cache as ocache
from tests.gpu_common import (assert_head_bit_exact, assert_within_tolerance, gpu_cache,
                              head_buffers, oracle_head, workload)

pytestmark = pytest.mark.gpu


def _decode(c, w):
    q = torch.from_numpy(w.q).cuda()
    out = kivi.decode_attn(c, q, w.config.sm_scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check_heads(c, w, heads, encode=True):
    out = _decode(c, w)
    G = w.config.group
    worst = (0.0, 0.0)
    for b, h in heads:
        ref_state = oracle_head(w, b, h)
        if encode:
            assert_head_bit_exact(head_buffers(c, b, h), ref_state, G)
        ref = ocache.decode_head(w.q[b, h], ref_state, w.config.sm_scale, G, w.bits)
        mx, rel = assert_within_tolerance(out[b, h], ref, f"b={b} h={h}")
        worst = (max(worst[0], mx), max(worst[1], rel))
    assert c.status_bits() == 0
    return worst


def test_tiny_single_head_prefill_and_decode():
    w = workload(1)
    c = gpu_cache(w)
    ref = ocache.Cache(1, 1, 128, 2, 32, 32, 256)
    ref.prefill(w.k, w.v, w.lengths, w.r_len)
    for name in ("k_codes", "v_codes"):
        assert np.array_equal(getattr(c, name).cpu().numpy().view(np.uint32), getattr(ref, name)), name
    for name in ("k_scale", "k_zero", "v_scale", "v_zero", "k_res", "v_res"):
        assert np.array_equal(getattr(c, name).cpu().numpy().view(np.uint16),
                              getattr(ref, name).view(np.uint16)), name
    out = _decode(c, w)
    assert_within_tolerance(out, ref.decode(w.q, w.config.sm_scale), "tiny")


def test_llama2_7b_layer_all_heads():
    w = workload(2)
    c = gpu_cache(w)
    heads = [(b, h) for b in range(8) for h in range(32)]
    _check_heads(c, w, heads)


def test_llama2_13b_layer_all_heads():
    w = workload(3)
    c = gpu_cache(w)
    heads = [(b, h) for b in range(16) for h in range(40)]
    _check_heads(c, w, heads, encode=False)
    sample = [(0, 0), (5, 17), (15, 39), (9, 3)]
    for b, h in sample:
        assert_head_bit_exact(head_buffers(c, b, h), oracle_head(w, b, h), 32)


def test_llama2_13b_layer_at_4_bits_sampled_heads():
    """640 (sequence, head) pairs at B=4: the decode with one sub-chunk in
    flight per wave (several workgroups per compute unit) at 4 bits."""
    w = workload(3, bits=4)
    c = gpu_cache(w)
    rng = np.random.default_rng(413)
    heads = sorted({(int(b), int(h)) for b, h in zip(rng.integers(0, 16, 24),
                                                     rng.integers(0, 40, 24))} | {(15, 39)})
    _check_heads(c, w, heads)


def test_llama2_13b_flush_of_full_window():
    """Flush of a full 128-token window per head: bit-exact against the
    oracle's bulk quantization of the same 2048 tokens, every head."""
    w = workload(3)
    c = gpu_cache(w)
    kivi.flush_residual(c)
    torch.cuda.synchronize()
    assert c.q_len.cpu().tolist() == [2048] * 16 and c.r_len.cpu().tolist() == [0] * 16
    kc = c.k_codes.cpu().numpy().view(np.uint32)
    vc = c.v_codes.cpu().numpy().view(np.uint32)
    ks, kz = c.k_scale.cpu().numpy(), c.k_zero.cpu().numpy()
    vs, vz = c.v_scale.cpu().numpy(), c.v_zero.cpu().numpy()
    for b in range(16):
        for h in range(40):
            enc = ocache.encode_tokens(w.k[b, h, 1920:2048], w.v[b, h, 1920:2048], 32, 2)
            assert np.array_equal(kc[b, h, 60:64], enc["k_codes"])
            assert np.array_equal(vc[b, h, 60:64], enc["v_codes"])
            assert np.array_equal(ks[b, h, 60:64].view(np.uint16), enc["k_scale"].view(np.uint16))
            assert np.array_equal(kz[b, h, 60:64].view(np.uint16), enc["k_zero"].view(np.uint16))
            assert np.array_equal(vs[b, h, 60:64].view(np.uint16), enc["v_scale"].view(np.uint16))
            assert np.array_equal(vz[b, h, 60:64].view(np.uint16), enc["v_zero"].view(np.uint16))
    assert c.status_bits() == 0
    assert not c.tickets.any()


def test_flush_only_full_windows_and_twice_in_a_row():
    """A batch where some windows are full: only those are flushed (lengths
    and codes), a second flush changes nothing, the tickets end at zero."""
    w = workload(3, batch=4)
    ql = np.array([1920, 1920, 1888, 1920], np.int32)
    rl = np.array([128, 5, 128, 0], np.int32)
    c = gpu_cache(w, q_len=ql, r_len=rl)
    before = c.k_codes.cpu().numpy().copy()
    for _ in range(2):
        kivi.flush_residual(c)
        torch.cuda.synchronize()
        assert c.q_len.cpu().tolist() == [2048, 1920, 2016, 1920]
        assert c.r_len.cpu().tolist() == [0, 5, 0, 0]
        assert not c.tickets.any() and c.status_bits() == 0
    after = c.k_codes.cpu().numpy()
    assert np.array_equal(after[1], before[1]) and np.array_equal(after[3], before[3])
    for b, h in [(0, 0), (0, 39), (2, 7)]:
        t0 = int(ql[b])
        enc = ocache.encode_tokens(w.k[b, h, t0:t0 + 128], w.v[b, h, t0:t0 + 128], 32, 2)
        assert np.array_equal(after[b, h, t0 // 32:t0 // 32 + 4].view(np.uint32), enc["k_codes"])


def test_flush_of_a_large_batch_with_few_full_windows():
    """Batch 64 x 32 heads: more flush units (two tiles of one (sequence,
    head)) than flush workgroups, so each workgroup takes several units in
    turn.  Only the sequences whose window is full move, bit for bit as the
    oracle encodes them; the rest keep their lengths and codes."""
    rng = np.random.default_rng(77)
    B, H, D, G, R, cap = 64, 32, 128, 32, 128, 512
    k = (rng.standard_normal((B, H, cap, D), np.float32) * 3).astype(np.float16)
    v = rng.standard_normal((B, H, cap, D), np.float32).astype(np.float16)
    ql = np.full(B, 256, np.int32)
    rl = rng.integers(0, R, B).astype(np.int32)
    full = np.zeros(B, bool)
    full[[0, 13, 40, 63]] = True
    rl[full] = R
    c = kivi.KiviCache(B, H, D, 2, G, R, cap)
    kivi.prefill(c, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                 torch.from_numpy(ql + rl).cuda(), torch.from_numpy(rl).cuda())
    torch.cuda.synchronize()
    before = c.k_codes.cpu().numpy().copy()
    kivi.flush_residual(c)
    torch.cuda.synchronize()
    assert np.array_equal(c.q_len.cpu().numpy(), np.where(full, ql + R, ql))
    assert np.array_equal(c.r_len.cpu().numpy(), np.where(full, 0, rl))
    assert not c.tickets.any() and c.status_bits() == 0
    after = c.k_codes.cpu().numpy()
    assert np.array_equal(after[~full], before[~full])
    for b, h in [(0, 0), (13, 31), (40, 7), (63, 16)]:
        enc = ocache.encode_tokens(k[b, h, 256:256 + R], v[b, h, 256:256 + R], G, 2)
        for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
            got = getattr(c, name)[b, h, 256 // G:(256 + R) // G].cpu().numpy()
            assert np.array_equal(got.view(np.uint8), enc[name].view(np.uint8)), (name, b, h)


def test_streaming_appends_and_flushes_match_prefill():
    """Token-by-token appends with a flush after each, on the GPU, give the
    same buffers as one GPU prefill and as the oracle's streaming cache."""
    w = workload(1)
    n = 200
    kt = torch.from_numpy(w.k).cuda()
    vt = torch.from_numpy(w.v).cuda()
    s = kivi.KiviCache(1, 1, 128, 2, 32, 32, 256)
    ref = ocache.Cache(1, 1, 128, 2, 32, 32, 256)
    for t in range(n):
        kivi.append_kv(s, kt[:, :, t].contiguous(), vt[:, :, t].contiguous())
        kivi.flush_residual(s)
        ref.append(w.k[:, :, t], w.v[:, :, t])
        ref.flush()
    torch.cuda.synchronize()
    b = kivi.KiviCache(1, 1, 128, 2, 32, 32, 256)
    kivi.prefill(b, kt, vt, torch.tensor([n], dtype=torch.int32, device="cuda"),
                 torch.tensor([n % 32], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert s.q_len.item() == 192 and s.r_len.item() == 8 and not s.tickets.any()
    for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
        g = getattr(s, name).cpu().numpy()
        assert np.array_equal(g, getattr(b, name).cpu().numpy()), name
        assert np.array_equal(g.view(np.uint8), getattr(ref, name).view(np.uint8)), name
    assert np.array_equal(s.k_res[0, 0, :8].cpu().numpy(), w.k[0, 0, 192:200])
    q = torch.from_numpy(w.q).cuda()
    out = kivi.decode_attn(s, q, w.config.sm_scale).cpu().numpy()
    assert_within_tolerance(out, ref.decode(w.q, w.config.sm_scale), "streamed")


@pytest.mark.parametrize("q_len,r_len", [
    (0, 0), (0, 1), (0, 32), (32, 0), (224, 0), (224, 32), (192, 31), (32, 1), (256, 0),
])
def test_edge_lengths(q_len, r_len):
    """Empty context, window only, quantized only, full capacity, full
    window, one token: each against the oracle."""
    w = workload(1)
    c = gpu_cache(w, q_len=[q_len], r_len=[r_len])
    out = _decode(c, w)
    st = ocache.head_state(w.k[0, 0], w.v[0, 0], q_len, r_len, 32, 2, 256, 32)
    ref = ocache.decode_head(w.q[0, 0], st, w.config.sm_scale, 32, 2)
    if q_len + r_len == 0:
        assert np.all(out == 0)
    else:
        assert_within_tolerance(out[0, 0], ref, f"{q_len}+{r_len}")
    assert_head_bit_exact(head_buffers(c, 0, 0), st, 32)


@pytest.mark.parametrize("capacity", [4096, 8192, 65536])
def test_split_count_does_not_change_the_result(capacity):
    """The same cache contents decoded with different capacities (hence
    different work splits: 8 to 64 splits, 1 to 2 chunks each) agree with
    the oracle."""
    w = workload(2, batch=2)
    c = gpu_cache(w, capacity=capacity)
    out = _decode(c, w)
    for b in range(2):
        for h in (0, 13, 31):
            ref = ocache.decode_head(w.q[b, h], oracle_head(w, b, h), 1.0, 32, 2)
            assert_within_tolerance(out[b, h], ref, f"cap {capacity}")


def test_decode_is_deterministic_and_leaves_workspace_clean():
    w = workload(2)
    c = gpu_cache(w)
    q = torch.from_numpy(w.q).cuda()
    first = kivi.decode_attn(c, q, 1.0).clone()
    for _ in range(10):
        again = kivi.decode_attn(c, q, 1.0)
        assert torch.equal(again, first)
    torch.cuda.synchronize()
    d = c.dims
    ws = c.workspace.cpu().numpy()
    bh = d.batch * d.heads
    tickets = ws[len(ws) - bh * 256:]
    assert np.all(tickets == 0)


def test_status_bits_and_skipped_sequences():
    w = workload(1)
    # append into a full window: dropped, flagged (capacity 224: no room to flush)
    c = gpu_cache(w, capacity=224, q_len=[224], r_len=[32])
    k1 = torch.from_numpy(w.k[:, :, 0]).cuda().contiguous()
    kivi.append_kv(c, k1, k1)
    torch.cuda.synchronize()
    assert c.r_len.item() == 32 and c.status_bits() == kivi.ST_RESIDUAL_FULL
    # flush past capacity: untouched, flagged
    c.clear_status()
    kivi.flush_residual(c)
    torch.cuda.synchronize()
    assert c.q_len.item() == 224 and c.r_len.item() == 32 and c.status_bits() == kivi.ST_CAPACITY
    # impossible lengths: output 0, flagged
    c.clear_status()
    c.q_len.fill_(33)
    out = _decode(c, w)
    assert np.all(out == 0) and c.status_bits() == kivi.ST_BAD_LENGTH
    c.clear_status()
    c.q_len.fill_(224)
    c.r_len.fill_(40)
    out = _decode(c, w)
    assert np.all(out == 0) and c.status_bits() == kivi.ST_BAD_LENGTH
    # prefill with a window that leaves a partial group: rejected
    c2 = kivi.KiviCache(1, 1, 128, 2, 32, 32, 256)
    kt = torch.from_numpy(w.k).cuda()
    kivi.prefill(c2, kt, kt, torch.tensor([100], dtype=torch.int32, device="cuda"),
                 torch.tensor([5], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert c2.q_len.item() == 0 and c2.status_bits() == kivi.ST_BAD_LENGTH
    # default window: len % G
    c3 = kivi.KiviCache(1, 1, 128, 2, 32, 32, 256)
    kivi.prefill(c3, kt, kt, torch.tensor([100], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert c3.q_len.item() == 96 and c3.r_len.item() == 4 and c3.status_bits() == 0


def test_workspace_too_small_is_rejected():
    w = workload(1)
    c = gpu_cache(w)
    q = torch.from_numpy(w.q).cuda()
    small = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(kivi.KiviError) as e:
        kivi.decode_attn(c, q, 1.0, workspace=small)
    assert e.value.code == kivi.KIVI_ENOSPC


def test_byte_model_matches_buffers():
    """The decode byte model counts exactly the cache bytes a decode reads."""
    w = workload(1)
    c = gpu_cache(w)
    per_head = wl.decode_bytes_per_head(224, 32, 128, 2, 32)
    k_codes = 224 * 128 * 2 // 8
    assert per_head == 2 * k_codes + 7 * 128 * 4 + 224 * 4 * 4 + 2 * 32 * 256 + 256 + 512
    assert c.nbytes() >= per_head - 768


def _near_tie_values(bits, rng, pairs=200):
    """(mn, mx, xs) triples of fp16 values for which (x - mn) / s (s the fp16
    step of a group with minimum mn and maximum mx, fp32 arithmetic) is a
    half-integer or within 2^-15 (2^-12 at B=8, whose quotients reach 255) of
    one: exact ties, and quotients near the rounding boundaries where a
    reciprocal-based shortcut could round the other way.  Negative minima
    give x - mn many significant bits."""
    levels = np.float32((1 << bits) - 1)
    f16 = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)
    f16 = np.concatenate([-f16[1:], f16])
    out = []
    for _ in range(pairs):
        mn = np.float16(-rng.uniform(0.5, 60.0))
        mx = np.float16(rng.uniform(0.5, 60.0))
        s = np.float32(np.float16((np.float32(mx) - np.float32(mn)) / levels))
        xs = f16[(f16 >= mn) & (f16 <= mx)]
        q = (xs.astype(np.float32) - np.float32(mn)) / s
        frac = np.abs(np.abs(q - np.rint(q)) - np.float32(0.5))
        near = xs[frac < (2.0 ** -15 if bits <= 4 else 2.0 ** -12)]
        if len(near):
            out.append((mn, mx, near))
    return out


def _near_tie_kv(bits, rng):
    """Keys and values of 2 heads x 128 tokens whose every group (key:
    channel over 32 tokens; value: token over 32 channels) holds its
    minimum, its maximum and 30 values at or near a rounding tie."""
    cases = _near_tie_values(bits, rng)
    assert sum(len(c[2]) for c in cases) > 300
    G, R, D, H = 32, 128, 128, 2
    k = np.zeros((1, H, R, D), np.float16)
    v = np.zeros((1, H, R, D), np.float16)
    for h in range(H):
        for g in range(R // G):
            for c in range(D):           # key group: channel c over tokens g*G .. g*G+G-1
                mn, mx, near = cases[rng.integers(len(cases))]
                col = np.concatenate([[mn, mx], rng.choice(near, size=G - 2)]).astype(np.float16)
                k[0, h, g * G:(g + 1) * G, c] = rng.permutation(col)
        for t in range(R):
            for j in range(D // G):      # value group: token t, channels j*G .. j*G+G-1
                mn, mx, near = cases[rng.integers(len(cases))]
                row = np.concatenate([[mn, mx], rng.choice(near, size=G - 2)]).astype(np.float16)
                v[0, h, t, j * G:(j + 1) * G] = rng.permutation(row)
    return k, v, G, R, D, H


def _assert_tiles_match_oracle(caches, k, v, G, R, H, bits):
    for h in range(H):
        enc = ocache.encode_tokens(k[0, h], v[0, h], G, bits)
        for c in caches:
            for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
                got = getattr(c, name)[0, h, :R // G].cpu().numpy()
                assert np.array_equal(got.view(np.uint8), enc[name].view(np.uint8)), name


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_quantizer_near_ties_bit_exact_on_both_encoders(bits):
    """Keys and values built from exact and near rounding ties: the prefill
    encoder and the flush kernel both match the oracle bit for bit."""
    rng = np.random.default_rng(77 + bits)
    k, v, G, R, D, H = _near_tie_kv(bits, rng)
    kt, vt = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    lens = torch.tensor([R], dtype=torch.int32, device="cuda")
    pre = kivi.KiviCache(1, H, D, bits, G, R, 256)
    kivi.prefill(pre, kt, vt, lens, torch.tensor([0], dtype=torch.int32, device="cuda"))
    fl = kivi.KiviCache(1, H, D, bits, G, R, 256)
    kivi.prefill(fl, kt, vt, lens, torch.tensor([R], dtype=torch.int32, device="cuda"))
    kivi.flush_residual(fl)
    torch.cuda.synchronize()
    assert pre.q_len.item() == R and fl.q_len.item() == R and fl.r_len.item() == 0
    _assert_tiles_match_oracle((pre, fl), k, v, G, R, H, bits)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_quantizer_near_ties_bit_exact_through_decode_step(bits):
    """The same near-tie keys and values flushed by kivi_decode_step: a
    window of R - 1 tokens, then a step that appends token R - 1 and so
    fills it (at B = 2 and 4 one kernel, which quantizes the window from
    its registers; at B = 8 the three kernels).  Bit for bit the oracle's."""
    rng = np.random.default_rng(77 + bits)
    k, v, G, R, D, H = _near_tie_kv(bits, rng)
    kt, vt = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    st = kivi.KiviCache(1, H, D, bits, G, R, 256)
    n = torch.tensor([R - 1], dtype=torch.int32, device="cuda")
    kivi.prefill(st, kt, vt, n, n)
    q = torch.from_numpy(rng.standard_normal((1, H, D)).astype(np.float16)).cuda()
    kivi.decode_step(st, kt[:, :, R - 1].contiguous(), vt[:, :, R - 1].contiguous(), q, 0.088)
    torch.cuda.synchronize()
    if bits != 8:
        assert kivi.decode_step_kernels(st.dims) == 1
    assert st.q_len.item() == R and st.r_len.item() == 0 and st.status_bits() == 0
    _assert_tiles_match_oracle((st,), k, v, G, R, H, bits)


def _state(c):
    return {n: t.cpu().numpy().copy() for n, t in c.buffers().items()}


def _step_both(make, k_new, v_new, q, scale):
    """Run append + decode + flush on one cache and decode_step on an
    identical one; return both outputs and both final states."""
    a, b = make(), make()
    kivi.append_kv(a, k_new, v_new)
    out_a = kivi.decode_attn(a, q, scale).clone()
    kivi.flush_residual(a)
    out_b = kivi.decode_step(b, k_new, v_new, q, scale).clone()
    torch.cuda.synchronize()
    return out_a, out_b, _state(a), _state(b)


def _assert_same_step(out_a, out_b, sa, sb):
    # the cache bit for bit; the output up to rounding: the whole-step kernel
    # may take the window tokens first, and the plain decode (two code words
    # per lane) sums in another lane order, fp32 sums of a few hundred terms
    # of up to |v| ~ 4 reordered (about 1e-5), through the softmax weights
    # (score sums reordered) up to about 1e-4
    torch.testing.assert_close(out_b, out_a, rtol=1e-4, atol=1e-4)
    for name in sa:
        assert np.array_equal(sa[name].view(np.uint8), sb[name].view(np.uint8)), name
    assert not sb["tickets"].any()


@pytest.mark.parametrize("q_len,r_len,capacity,bad_q", [
    (192, 31, 256, None),   # the append fills the window: flushed in the same kernel
    (192, 5, 256, None),    # append only
    (0, 0, 256, None),      # empty cache
    (192, 32, 256, None),   # full window: the append is refused, the flush happens
    (192, 31, 224, None),   # the flush would pass capacity
    (192, 31, 256, 33),     # q_len not a multiple of G
])
def test_decode_step_matches_three_calls_tiny(q_len, r_len, capacity, bad_q):
    w = workload(1)
    kn = torch.from_numpy(w.k[:, :, 255]).cuda().contiguous()
    vn = torch.from_numpy(w.v[:, :, 255]).cuda().contiguous()
    q = torch.from_numpy(w.q).cuda()

    def make():
        c = gpu_cache(w, capacity=capacity, q_len=[q_len], r_len=[r_len])
        if bad_q is not None:
            c.q_len.fill_(bad_q)
        return c
    out_a, out_b, sa, sb = _step_both(make, kn, vn, q, w.config.sm_scale)
    _assert_same_step(out_a, out_b, sa, sb)


@pytest.mark.parametrize("bits,G,R", [
    (2, 32, 128), (4, 32, 128), (2, 64, 128), (4, 128, 128),
    (2, 32, 64), (4, 64, 64),        # 8 window tokens per wave
    (2, 32, 256), (4, 128, 256),     # longer windows: read again and quantized through LDS
])
def test_decode_step_flush_in_kernel_matches_oracle(bits, G, R):
    """The append fills the window and the same kernel flushes it: the new
    tiles equal the oracle's encoding of the window (new token included) bit
    for bit, and the whole state equals that of the three separate calls."""
    rng = np.random.default_rng(1000 + 7 * bits + G + R)
    B, H, D = 2, 3, 128
    ql, n = G, G + R - 1
    cap = ql + R
    k = rng.standard_normal((B, H, n, D), np.float32)
    k[..., ::9] *= 8.0                                  # a few outlier key channels
    k = k.astype(np.float16)
    v = rng.standard_normal((B, H, n, D), np.float32).astype(np.float16)
    k_new = rng.standard_normal((B, H, D), np.float32).astype(np.float16)
    v_new = rng.standard_normal((B, H, D), np.float32).astype(np.float16)
    q = rng.standard_normal((B, H, D), np.float32).astype(np.float16)
    kt, vt = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    lens = torch.full((B,), n, dtype=torch.int32, device="cuda")
    res = torch.full((B,), R - 1, dtype=torch.int32, device="cuda")

    def make():
        c = kivi.KiviCache(B, H, D, bits, G, R, cap)
        kivi.prefill(c, kt, vt, lens, res)
        return c
    dims = kivi.make_dims(batch=B, heads=H, head_dim=D, bits=bits, group=G, residual=R,
                          capacity=cap)
    assert kivi.decode_splits(dims) == 1
    out_a, out_b, sa, sb = _step_both(make, torch.from_numpy(k_new).cuda(),
                                      torch.from_numpy(v_new).cuda(), torch.from_numpy(q).cuda(),
                                      0.125)
    _assert_same_step(out_a, out_b, sa, sb)
    assert (sb["q_len"] == ql + R).all() and (sb["r_len"] == 0).all()
    assert not sb["status"].any()
    t0, t1 = ql // G, (ql + R) // G
    for b in range(B):
        for h in range(H):
            enc = ocache.encode_tokens(np.concatenate([k[b, h, ql:], k_new[b, h][None]]),
                                       np.concatenate([v[b, h, ql:], v_new[b, h][None]]), G, bits)
            for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
                got = sb[name][b, h, t0:t1]
                assert np.array_equal(got.view(np.uint8), enc[name].view(np.uint8)), (name, b, h)


@pytest.mark.parametrize("bits,G,R", [
    (2, 32, 128), (4, 32, 128), (2, 64, 128), (4, 64, 128), (2, 128, 128), (4, 128, 128),
    (2, 32, 96), (2, 64, 64), (4, 32, 32),     # windows shorter than 128: idle key/value waves
    (8, 32, 128), (2, 32, 256), (4, 64, 256),  # the tile-staging flush (B = 8, R > 128)
])
def test_flush_kernel_matches_oracle_across_shapes(bits, G, R):
    """kivi_flush_residual alone on full windows of every shape its two
    kernels take (key waves and value waves for B = 2, 4 and R <= 128, with
    the key waves of a G > 32 tile merging through LDS; tile staging
    otherwise): the new tiles equal the oracle's encoding of the window bit
    for bit, the lengths move by R and nothing else is touched."""
    rng = np.random.default_rng(2000 + 7 * bits + G + R)
    B, H, D = 3, 5, 128
    ql = 2 * G
    n, cap = ql + R, ql + R + G
    k = rng.standard_normal((B, H, n, D), np.float32)
    k[..., ::7] *= 16.0                                 # outlier key channels
    k[..., 5] += 40.0                                   # and one far from zero
    k = k.astype(np.float16)
    v = rng.standard_normal((B, H, n, D), np.float32).astype(np.float16)
    c = kivi.KiviCache(B, H, D, bits, G, R, cap)
    kivi.prefill(c, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                 torch.full((B,), n, dtype=torch.int32, device="cuda"),
                 torch.full((B,), R, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    before = {name: t.cpu().numpy().copy() for name, t in c.buffers().items()}
    kivi.flush_residual(c)
    torch.cuda.synchronize()
    after = {name: t.cpu().numpy() for name, t in c.buffers().items()}
    assert c.status_bits() == 0
    assert (after["q_len"] == ql + R).all() and (after["r_len"] == 0).all()
    t0, t1 = ql // G, (ql + R) // G
    for b in range(B):
        for h in range(H):
            enc = ocache.encode_tokens(k[b, h, ql:], v[b, h, ql:], G, bits)
            for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
                got = after[name][b, h, t0:t1]
                assert np.array_equal(got.view(np.uint8), enc[name].view(np.uint8)), (name, b, h)
                # tiles before and after the window's are untouched
                assert np.array_equal(after[name][b, h, :t0].view(np.uint8),
                                      before[name][b, h, :t0].view(np.uint8)), (name, b, h)
                assert np.array_equal(after[name][b, h, t1:].view(np.uint8),
                                      before[name][b, h, t1:].view(np.uint8)), (name, b, h)


@pytest.mark.parametrize("number", [2, 4])
def test_decode_step_matches_three_calls_full_workloads(number):
    """The Llama-2-7B-shaped layer (every window fills and is flushed in the
    step) and a ragged batch of 8 (a mix of flushed and not): one kernel per
    step (one workgroup per (sequence, head), 256 workgroups), identical to
    the three calls."""
    w = workload(number, batch=8 if number == 4 else None)
    cfg = w.config
    rl = np.minimum(w.r_len, cfg.residual - 1) if number == 4 else w.r_len - 1
    rng = np.random.default_rng(5)
    kn = torch.from_numpy(rng.standard_normal((len(rl), cfg.heads, 128), np.float32)
                          .astype(np.float16)).cuda()
    vn = torch.from_numpy(rng.standard_normal((len(rl), cfg.heads, 128), np.float32)
                          .astype(np.float16)).cuda()
    q = torch.from_numpy(w.q).cuda()
    d = w.dims()
    assert kivi.decode_splits(kivi.make_dims(**d)) == 1
    out_a, out_b, sa, sb = _step_both(lambda: gpu_cache(w, r_len=rl), kn, vn, q, cfg.sm_scale)
    _assert_same_step(out_a, out_b, sa, sb)
    if number == 2:
        assert (sb["r_len"] == 0).all() and (sb["q_len"] == w.q_len + 128).all()


def test_decode_step_on_a_large_grid_matches_three_calls():
    """More (sequence, head) pairs than compute units (the 13B layer, 640):
    the decode runs with one sub-chunk in flight per wave so that several
    workgroups share a compute unit, and decode_step launches the three
    kernels; the result is that of the three calls and the window flushes."""
    w = workload(3)
    cfg = w.config
    rl = w.r_len - 1
    rng = np.random.default_rng(8)
    kn = torch.from_numpy(rng.standard_normal((len(rl), cfg.heads, 128), np.float32)
                          .astype(np.float16)).cuda()
    vn = torch.from_numpy(rng.standard_normal((len(rl), cfg.heads, 128), np.float32)
                          .astype(np.float16)).cuda()
    q = torch.from_numpy(w.q).cuda()
    out_a, out_b, sa, sb = _step_both(lambda: gpu_cache(w, r_len=rl), kn, vn, q, cfg.sm_scale)
    _assert_same_step(out_a, out_b, sa, sb)
    assert (sb["r_len"] == 0).all() and (sb["q_len"] == w.q_len + 128).all()


def test_decode_step_streaming_matches_oracle():
    """Consecutive whole steps in one kernel each, over two sequences whose
    windows fill at different steps (one flush per sequence along the way):
    every step's output against the oracle's append, decode, flush, and the
    final buffers bit for bit; the tickets are left at zero after each."""
    rng = np.random.default_rng(4242)
    B, H, D, G, R, bits = 2, 3, 128, 32, 64, 2
    cap = 4 * G + R
    n0 = np.array([G + R - 3, 2 * G + R - 7])       # windows 3 and 7 short of full
    res = np.array([R - 3, R - 7])
    T = int(n0.max())
    k = rng.standard_normal((B, H, T, D), np.float32)
    k[..., 5] *= 40.0                                # an outlier key channel
    k = k.astype(np.float16)
    v = rng.standard_normal((B, H, T, D), np.float32).astype(np.float16)
    c = kivi.KiviCache(B, H, D, bits, G, R, cap)
    kivi.prefill(c, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                 torch.from_numpy(n0.astype(np.int32)).cuda(),
                 torch.from_numpy(res.astype(np.int32)).cuda())
    assert kivi.decode_step_kernels(c.dims) == 1
    ref = ocache.Cache(B, H, D, bits, G, R, cap)
    ref.prefill(k, v, n0, res)
    ws = kivi.new_workspace(c.dims)
    for step in range(10):
        kn = rng.standard_normal((B, H, D), np.float32).astype(np.float16)
        vn = rng.standard_normal((B, H, D), np.float32).astype(np.float16)
        q = (rng.standard_normal((B, H, D), np.float32) / np.sqrt(D)).astype(np.float16)
        out = kivi.decode_step(c, torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(),
                               torch.from_numpy(q).cuda(), 1.0, workspace=ws)
        ref.append(kn, vn)
        expect = ref.decode(q, 1.0)
        ref.flush()
        torch.cuda.synchronize()
        assert_within_tolerance(out.cpu().numpy(), expect, f"step {step}")
        assert not c.tickets.any() and c.status_bits() == 0
    assert np.array_equal(c.q_len.cpu().numpy(), ref.q_len)
    assert np.array_equal(c.r_len.cpu().numpy(), ref.r_len)
    for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
        assert np.array_equal(getattr(c, name).cpu().numpy().view(np.uint8),
                              getattr(ref, name).view(np.uint8)), name


def test_decode_step_with_split_heads_uses_three_kernels():
    """Batch 1 x 32 heads over a long context splits each (sequence, head)
    over several workgroups; decode_step then runs the three kernels."""
    w = workload(5, bits=2)
    d = w.dims()
    assert kivi.decode_splits(kivi.make_dims(**d)) > 1
    ql, rl = np.array([4096], np.int32), np.array([127], np.int32)
    rng = np.random.default_rng(6)
    kn = torch.from_numpy(rng.standard_normal((1, 32, 128), np.float32).astype(np.float16)).cuda()
    vn = torch.from_numpy(rng.standard_normal((1, 32, 128), np.float32).astype(np.float16)).cuda()
    q = torch.from_numpy(w.q).cuda()
    out_a, out_b, sa, sb = _step_both(lambda: gpu_cache(w, q_len=ql, r_len=rl), kn, vn, q, 1.0)
    _assert_same_step(out_a, out_b, sa, sb)


# ------------------------------------------------------------------ 8 bits
# The tutorial's parameter section lists 2, 4 and 8 bits.  At B=8 a word
# holds four channels, so a token spans 32 lanes.

def test_eight_bit_llama2_7b_shape_all_heads():
    """Two sequences of the Llama-2-7B-shaped layer at B=8: every cache buffer
    bit for bit and every head's output against the oracle.  64 (sequence,
    head) pairs are split four ways, so the split merge runs at B=8 too."""
    w = workload(2, bits=8, batch=2)
    c = gpu_cache(w)
    assert kivi.decode_splits(kivi.make_dims(**w.dims())) == 4
    worst = _check_heads(c, w, [(b, h) for b in range(2) for h in range(32)])
    assert worst[0] < 2e-3


def test_eight_bit_flush_and_step_match_oracle():
    """At B=8 the whole step is the three kernels; after appending the last
    window token the flush quantizes the full 128-token window bit for bit as
    the oracle does, and the step's output matches the oracle's decode."""
    w = workload(3, bits=8, batch=2)
    cfg = w.config
    d = w.dims()
    assert kivi.decode_step_kernels(kivi.make_dims(**d)) == 3
    rl = w.r_len - 1
    b_idx = np.arange(2)
    last = w.q_len + rl
    kn = np.ascontiguousarray(w.k[b_idx, :, last])
    vn = np.ascontiguousarray(w.v[b_idx, :, last])
    q = torch.from_numpy(w.q).cuda()
    out_a, out_b, sa, sb = _step_both(lambda: gpu_cache(w, r_len=rl), torch.from_numpy(kn).cuda(),
                                      torch.from_numpy(vn).cuda(), q, cfg.sm_scale)
    _assert_same_step(out_a, out_b, sa, sb)
    assert (sb["r_len"] == 0).all() and (sb["q_len"] == w.q_len + 128).all()
    out = out_b.cpu().numpy()
    G = cfg.group
    for b in range(2):
        for h in (0, 17, 39):
            t0 = int(w.q_len[b])
            enc = ocache.encode_tokens(w.k[b, h, t0:t0 + 128], w.v[b, h, t0:t0 + 128], G, 8)
            for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
                got = sb[name][b, h, t0 // G:(t0 + 128) // G]
                assert np.array_equal(got.view(np.uint8), enc[name].view(np.uint8)), (name, b, h)
            ref = ocache.decode_head(w.q[b, h], oracle_head(w, b, h), cfg.sm_scale, G, 8)
            assert_within_tolerance(out[b, h], ref, f"b={b} h={h}")


@pytest.mark.parametrize("q_len,r_len", [(0, 1), (32, 0), (32, 1), (4064, 31), (3968, 128)])
def test_eight_bit_edge_lengths(q_len, r_len):
    w = workload(2, bits=8, batch=1)
    c = gpu_cache(w, q_len=[q_len], r_len=[r_len])
    out = _decode(c, w)
    for h in (0, 31):
        st = ocache.head_state(w.k[0, h], w.v[0, h], q_len, r_len, 32, 8, 4096, 128)
        ref = ocache.decode_head(w.q[0, h], st, 1.0, 32, 8)
        assert_within_tolerance(out[0, h], ref, f"{q_len}+{r_len}")
        assert_head_bit_exact(head_buffers(c, 0, h), st, 32)


D_HEAD = 128
_MODES = ("rise", "spike", "fall", "steps")


def _score_profile_kv(mode, T, rng):
    """Keys whose log2 scores against the unit query q follow a profile along
    the sequence (before quantization): 'rise' climbs 60 over the sequence,
    'fall' descends 60, 'steps' climbs 9 every 512 tokens, 'spike' is noise
    with one token 40 above it in the last quarter and one 25 above it near
    the end.  The noise is N(0, 1) in every channel."""
    q = rng.standard_normal(D_HEAD)
    q /= np.linalg.norm(q)
    t = np.arange(T, dtype=np.float64)
    if mode == "rise":
        s = 60.0 * t / T
    elif mode == "fall":
        s = 60.0 * (1.0 - t / T)
    elif mode == "steps":
        s = 9.0 * (t // 512)
    else:
        s = np.zeros(T)
        s[int(rng.integers(3 * T // 4, T - 200))] = 40.0
        s[T - 3] = 25.0
    k = np.outer(s / np.log2(np.e), q) + rng.standard_normal((T, D_HEAD))
    v = rng.standard_normal((T, D_HEAD))
    return q.astype(np.float16), k.astype(np.float16), v.astype(np.float16)


@pytest.mark.parametrize("shape", ["one_word_lanes", "two_word_lanes", "split_heads",
                                   "step_fills_window", "step_appends"])
def test_score_profiles_that_move_the_softmax_reference(shape):
    """Score profiles that make the online softmax move its reference often
    (a steady climb, steps of 9 in log2 units, a late spike) or never after
    the start (a fall), through the one-word-per-lane decode (one workgroup
    per (sequence, head)), the two-word-lane decode (long caches), the
    decode split over many workgroups (merged by log-sum-exp), and the
    one-kernel step, whose append either fills the window (the window's
    tokens then go before the quantized stream) or not: sampled heads
    against the oracle's fp64 softmax over every token."""
    R, G, bits = 128, 32, 2
    step = shape.startswith("step")
    if shape in ("one_word_lanes", "step_fills_window"):
        batch, heads, cap, ql = 8, 32, 4096, 3968
    elif shape == "step_appends":
        batch, heads, cap, ql = 8, 32, 4096, 3840
    elif shape == "two_word_lanes":
        batch, heads, cap, ql = 8, 32, 16384, 4096
    else:
        batch, heads, cap, ql = 1, 4, 65536, 32768
    win = {"step_fills_window": R, "step_appends": 100}.get(shape, R - 1)  # after the step
    T = ql + win
    rng = np.random.default_rng(70 + ["one_word_lanes", "two_word_lanes", "split_heads",
                                      "step_fills_window", "step_appends"].index(shape))
    k = np.empty((batch, heads, T, D_HEAD), np.float16)
    v = np.empty_like(k)
    q = np.empty((batch, heads, D_HEAD), np.float16)
    modes = {}
    for b in range(batch):
        for h in range(heads):
            modes[b, h] = _MODES[(b * heads + h) % len(_MODES)]
            q[b, h], k[b, h], v[b, h] = _score_profile_kv(modes[b, h], T, rng)
    c = kivi.KiviCache(batch, heads, D_HEAD, bits, G, R, cap)
    splits = kivi.decode_splits(c.dims)
    assert (splits > 1) == (shape == "split_heads"), splits
    lens = np.full(batch, T - step, np.int32)
    wins = np.full(batch, win - step, np.int32)
    kivi.prefill(c, torch.from_numpy(k[:, :, :T - step]).cuda(),
                 torch.from_numpy(v[:, :, :T - step]).cuda(),
                 torch.from_numpy(lens).cuda(), torch.from_numpy(wins).cuda())
    qt = torch.from_numpy(q).cuda()
    if step:
        assert kivi.decode_step_kernels(c.dims) == 1
        kn = torch.from_numpy(np.ascontiguousarray(k[:, :, T - 1])).cuda()
        vn = torch.from_numpy(np.ascontiguousarray(v[:, :, T - 1])).cuda()
        out = kivi.decode_step(c, kn, vn, qt, 1.0).cpu().numpy()
    else:
        out = kivi.decode_attn(c, qt, 1.0).cpu().numpy()
    assert c.status_bits() == 0
    picks = [(b, h) for b in range(batch) for h in range(heads)]
    if len(picks) > 16:  # two heads per sequence, every profile among them
        picks = [(b, (b + j) % heads) for b in range(batch) for j in (0, 1)]
    for b, h in picks:
        st = ocache.head_state(k[b, h], v[b, h], ql, win, G, bits, cap, R)
        ref = ocache.decode_head(q[b, h], st, 1.0, G, bits)
        assert_within_tolerance(out[b, h], ref, f"{shape} b={b} h={h} {modes[b, h]}")
