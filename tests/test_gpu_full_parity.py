"""GPU parity at full workload size on every (sequence, head), through the C ABI.

* The long-context workload (1 x 32 heads, 130944 quantized + 128 window
  tokens, G = 128) at B = 2, 4 and 8: every head's codes, zero-points and
  steps bit for bit, every head's decode (8 splits per head, merged) against
  the oracle's fp64 attention.  The decode runs on a workspace that held
  garbage and went through kivi_workspace_init.
* The ragged batch-64 workload (2048 (sequence, head) pairs, contexts
  1024..8192, windows 0..127): every head bit for bit and to tolerance.
* The one-kernel step (kivi_decode_step) on the Llama-2-7B-shaped layer,
  directly against the oracle's append, decode and flush: every head's
  output and the whole cache after the step, for a step whose append fills
  the window (flushed from registers) and one that does not.
* The step's register flush on exact and near rounding ties (the inputs of
  the near-tie encoder test), bit for bit against the oracle's quantizer.
* Counters that did not start at zero are reported (KIVI_ST_TICKETS), and
  kivi_cache_init / kivi_workspace_init make a cache and a workspace usable.

Tolerance of the decode: max-abs 2e-3 and relative L2 1e-3 against the fp64
oracle on the same dequantized values.  The oracle runs on a pool of threads.
"""

import numpy as np
import pytest
import torch

from bit_kv_cache_decode_amd import kivi
from oracle import cache as ocache
from tests.gpu_common import (assert_head_bit_exact, assert_within_tolerance, gpu_cache,
                              head_of, host_buffers, oracle_head, parallel_map, workload)
from tests.test_gpu_parity import _near_tie_values

pytestmark = pytest.mark.gpu


def _all_heads(w):
    return [(b, h) for b in range(w.q.shape[0]) for h in range(w.q.shape[1])]


def _check_all(c, w, out, heads, bit_exact=True):
    """Every listed head against the oracle (its own encoding of the same
    fp16 tokens); returns the worst (max-abs, rel-L2)."""
    host = host_buffers(c) if bit_exact else None
    G = w.config.group

    def one(bh):
        b, h = bh
        st = oracle_head(w, b, h)
        if bit_exact:
            assert_head_bit_exact(head_of(host, b, h), st, G)
        ref = ocache.decode_head(w.q[b, h], st, w.config.sm_scale, G, w.bits)
        return assert_within_tolerance(out[b, h], ref, f"b={b} h={h}")

    res = parallel_map(one, heads)
    return max(r[0] for r in res), max(r[1] for r in res)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_long_context_every_head(bits):
    w = workload(5, bits=bits)
    c = gpu_cache(w)
    dims = c.dims
    assert kivi.decode_splits(dims) > 1
    print(f"long context B={bits}: {kivi.decode_splits(dims)} splits per head", flush=True)
    ws = torch.full((kivi.workspace_bytes(dims),), 0xA5, dtype=torch.uint8, device="cuda")
    kivi.workspace_init(dims, ws)
    out = kivi.decode_attn(c, torch.from_numpy(w.q).cuda(), w.config.sm_scale, workspace=ws)
    torch.cuda.synchronize()
    assert c.status_bits() == 0
    worst = _check_all(c, w, out.cpu().numpy(), _all_heads(w))
    print(f"long context B={bits}: worst max-abs {worst[0]:.2e}, rel-L2 {worst[1]:.2e}")


def test_ragged_serving_every_head():
    w = workload(4)
    c = gpu_cache(w)
    assert np.array_equal(c.q_len.cpu().numpy(), w.q_len)
    assert np.array_equal(c.r_len.cpu().numpy(), w.r_len)
    out = kivi.decode_attn(c, torch.from_numpy(w.q).cuda(), w.config.sm_scale)
    torch.cuda.synchronize()
    assert c.status_bits() == 0
    worst = _check_all(c, w, out.cpu().numpy(), _all_heads(w))
    print(f"ragged batch 64: worst max-abs {worst[0]:.2e}, rel-L2 {worst[1]:.2e}")


def test_two_word_lanes_every_head_with_half_sub_chunks():
    """The 7B-shaped batch in a cache of capacity 8192: one workgroup per
    (sequence, head) and, by capacity, 16 sub-chunks of 64 tokens per wave,
    which the decode takes with two code words per lane.  Every second
    sequence holds 32 fewer quantized tokens, so its last sub-chunk has one
    valid tile (the masked case).  Every head against the oracle."""
    w = workload(2)
    cap = 8192
    ql = w.q_len.copy()
    ql[1::2] -= 32
    rl = w.r_len.copy()
    c = gpu_cache(w, capacity=cap, q_len=ql, r_len=rl)
    assert kivi.decode_splits(c.dims) == 1
    out = kivi.decode_attn(c, torch.from_numpy(w.q).cuda(), w.config.sm_scale).cpu().numpy()
    assert c.status_bits() == 0
    cfg = w.config

    def one(bh):
        b, h = bh
        st = ocache.head_state(w.k[b, h], w.v[b, h], int(ql[b]), int(rl[b]), cfg.group, w.bits,
                               cap, cfg.residual)
        ref = ocache.decode_head(w.q[b, h], st, cfg.sm_scale, cfg.group, w.bits)
        return assert_within_tolerance(out[b, h], ref, f"b={b} h={h} q_len={ql[b]}")

    parallel_map(one, _all_heads(w))


@pytest.mark.parametrize("fills", [True, False])
def test_whole_step_kernel_llama2_7b_every_head_against_oracle(fills):
    """kivi_decode_step (one kernel) appends token t of every (sequence, head)
    to a cache holding tokens [0, t): 3968 quantized plus 127 window tokens
    (the append fills the window and the kernel flushes it) or plus 100
    (append only).  The output of every head is compared with the oracle's
    decode over tokens [0, t]; the cache after the step with the oracle's
    cache holding the same tokens, bit for bit."""
    w = workload(2)
    cfg = w.config
    B, H = w.q.shape[:2]
    ql = w.q_len.astype(np.int32)
    rl = (w.r_len - 1 if fills else np.full(B, 100)).astype(np.int32)
    c = gpu_cache(w, q_len=ql, r_len=rl)
    assert kivi.decode_step_kernels(c.dims) == 1
    last = ql + rl
    k_new = torch.from_numpy(np.ascontiguousarray(w.k[np.arange(B), :, last])).cuda()
    v_new = torch.from_numpy(np.ascontiguousarray(w.v[np.arange(B), :, last])).cuda()
    out = kivi.decode_step(c, k_new, v_new, torch.from_numpy(w.q).cuda(), cfg.sm_scale)
    torch.cuda.synchronize()
    assert c.status_bits() == 0 and not c.tickets.any()
    out = out.cpu().numpy()
    host = host_buffers(c)
    G, R = cfg.group, cfg.residual
    q_after = ql + R if fills else ql
    r_after = np.zeros(B, np.int32) if fills else rl + 1
    assert np.array_equal(host["q_len"], q_after) and np.array_equal(host["r_len"], r_after)

    def one(bh):
        b, h = bh
        before_flush = ocache.head_state(w.k[b, h], w.v[b, h], int(ql[b]), int(rl[b]) + 1, G,
                                         w.bits, cfg.capacity, R)
        ref = ocache.decode_head(w.q[b, h], before_flush, cfg.sm_scale, G, w.bits)
        after = ocache.head_state(w.k[b, h], w.v[b, h], int(q_after[b]), int(r_after[b]), G,
                                  w.bits, cfg.capacity, R)
        assert_head_bit_exact(head_of(host, b, h), after, G)
        return assert_within_tolerance(out[b, h], ref, f"b={b} h={h}")

    res = parallel_map(one, _all_heads(w))
    print(f"whole step ({'flush' if fills else 'append only'}): worst max-abs "
          f"{max(r[0] for r in res):.2e}, rel-L2 {max(r[1] for r in res):.2e}")


@pytest.mark.parametrize("bits", [2, 4])
def test_whole_step_register_flush_on_near_ties(bits):
    """Window keys and values built from exact and near rounding ties (as in
    the near-tie encoder test); the step appends the 128th window token and
    quantizes the window from the registers that hold it for the attention.
    The new tiles equal the oracle's encoding bit for bit."""
    rng = np.random.default_rng(177 + bits)
    cases = _near_tie_values(bits, rng)
    G, R, D, H, ql = 32, 128, 128, 4, 64
    k = np.zeros((1, H, ql + R, D), np.float16)
    v = np.zeros((1, H, ql + R, D), np.float16)
    k[0, :, :ql] = rng.standard_normal((H, ql, D)).astype(np.float16)
    v[0, :, :ql] = rng.standard_normal((H, ql, D)).astype(np.float16)
    for h in range(H):
        for g in range(R // G):
            for ch in range(D):          # key group: channel ch over G window tokens
                mn, mx, near = cases[rng.integers(len(cases))]
                col = np.concatenate([[mn, mx], rng.choice(near, size=G - 2)]).astype(np.float16)
                k[0, h, ql + g * G:ql + (g + 1) * G, ch] = rng.permutation(col)
        for t in range(R):
            for j in range(D // G):      # value group: window token t, channels j*G ..
                mn, mx, near = cases[rng.integers(len(cases))]
                row = np.concatenate([[mn, mx], rng.choice(near, size=G - 2)]).astype(np.float16)
                v[0, h, ql + t, j * G:(j + 1) * G] = rng.permutation(row)
    c = kivi.KiviCache(1, H, D, bits, G, R, ql + R)
    kivi.prefill(c, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                 torch.tensor([ql + R - 1], dtype=torch.int32, device="cuda"),
                 torch.tensor([R - 1], dtype=torch.int32, device="cuda"))
    assert kivi.decode_step_kernels(c.dims) == 1
    q = torch.from_numpy((rng.standard_normal((1, H, D)) / np.sqrt(D)).astype(np.float16)).cuda()
    kivi.decode_step(c, torch.from_numpy(np.ascontiguousarray(k[:, :, -1])).cuda(),
                     torch.from_numpy(np.ascontiguousarray(v[:, :, -1])).cuda(), q, 1.0)
    torch.cuda.synchronize()
    assert c.q_len.item() == ql + R and c.r_len.item() == 0 and c.status_bits() == 0
    host = host_buffers(c)
    for h in range(H):
        enc = ocache.encode_tokens(k[0, h, ql:], v[0, h, ql:], G, bits)
        for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
            got = host[name][0, h, ql // G:(ql + R) // G]
            assert np.array_equal(got.view(np.uint8), enc[name].view(np.uint8)), (name, h)


# ---------------------------------------------------------- counters and init

def test_uninitialised_workspace_is_reported_and_init_repairs_it():
    """A split decode (capacity 65536: several workgroups per (sequence,
    head)) on a workspace full of 0xFF bytes: the merge cannot find its last
    workgroup, which KIVI_ST_TICKETS reports; after kivi_workspace_init the
    same workspace gives the oracle's output and stays clean."""
    w = workload(2, batch=2)
    c = gpu_cache(w, capacity=65536)
    dims = c.dims
    assert kivi.decode_splits(dims) > 1
    ws = torch.full((kivi.workspace_bytes(dims),), 0xFF, dtype=torch.uint8, device="cuda")
    q = torch.from_numpy(w.q).cuda()
    kivi.decode_attn(c, q, 1.0, workspace=ws)
    torch.cuda.synchronize()
    assert c.status_bits() & kivi.ST_TICKETS
    c.clear_status()
    kivi.workspace_init(dims, ws)
    out = kivi.decode_attn(c, q, 1.0, workspace=ws)
    torch.cuda.synchronize()
    assert c.status_bits() == 0
    out = out.cpu().numpy()
    for b, h in [(0, 0), (1, 17), (1, 31)]:
        ref = ocache.decode_head(w.q[b, h], oracle_head(w, b, h, capacity=65536), 1.0, 32, 2)
        assert_within_tolerance(out[b, h], ref, f"b={b} h={h}")
    again = kivi.decode_attn(c, q, 1.0, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(again.cpu(), torch.from_numpy(out)) and c.status_bits() == 0
    small = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(kivi.KiviError) as e:
        kivi.workspace_init(dims, small)
    assert e.value.code == kivi.KIVI_ENOSPC


@pytest.mark.parametrize("entry", ["flush", "step"])
def test_uninitialised_cache_tickets_are_reported_and_cache_init_empties(entry):
    """Ticket counters that do not start at zero: the flush (and the
    one-kernel step) cannot find the workgroup that commits the lengths, so
    the lengths stay and KIVI_ST_TICKETS is set.  kivi_cache_init then
    leaves an empty cache (lengths, counters and status zero) that works."""
    w = workload(1)
    c = gpu_cache(w, q_len=[224], r_len=[32 if entry == "flush" else 31])
    c.tickets.fill_(5)
    if entry == "flush":
        kivi.flush_residual(c)
    else:
        assert kivi.decode_step_kernels(c.dims) == 1
        kn = torch.from_numpy(w.k[:, :, 255]).cuda().contiguous()
        kivi.decode_step(c, kn, kn, torch.from_numpy(w.q).cuda(), w.config.sm_scale)
    torch.cuda.synchronize()
    assert c.status_bits() & kivi.ST_TICKETS
    assert c.q_len.item() == 224
    kivi.cache_init(c)
    torch.cuda.synchronize()
    assert c.q_len.item() == 0 and c.r_len.item() == 0 and c.status_bits() == 0
    assert not c.tickets.any()
    kt = torch.from_numpy(w.k).cuda()
    vt = torch.from_numpy(w.v).cuda()
    for t in range(40):   # appends and one flush on the emptied cache
        kivi.append_kv(c, kt[:, :, t].contiguous(), vt[:, :, t].contiguous())
        kivi.flush_residual(c)
    torch.cuda.synchronize()
    assert c.q_len.item() == 32 and c.r_len.item() == 8 and c.status_bits() == 0
    st = ocache.head_state(w.k[0, 0], w.v[0, 0], 32, 8, 32, 2, 256, 32)
    out = kivi.decode_attn(c, torch.from_numpy(w.q).cuda(), w.config.sm_scale)
    ref = ocache.decode_head(w.q[0, 0], st, w.config.sm_scale, 32, 2)
    assert_within_tolerance(out.cpu().numpy()[0, 0], ref, "after cache_init")
