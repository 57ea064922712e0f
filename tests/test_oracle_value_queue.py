"""Pins of the value-queue oracle (discosf KIVI tutorial, section 3.2: values
enter an fp16 queue and leave it oldest first, quantized one token at a time
once more than R are queued; keys keep the window flush of section 3.1).

Each test ties ``oracle.value_queue`` to something other than itself: the bulk
quantizer (per-token value groups carry no state, so a value quantized on
its way out of the queue has the bulk codes), the queue of
``oracle.cache.value_queue`` (already pinned to the bulk quantizer), a
hand-listed token layout, and the plain fp16 attention of a queue that has
not overflowed.  A second part plants plausible mistakes and checks that a
pin catches each.
"""

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import cache as ocache
from oracle import quantizer as oq
from oracle import value_queue as ovq

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _draw(rng, B, H, n, D):
    k = rng.standard_normal((B, H, n, D)).astype(np.float32)
    k[..., 3] *= 30.0
    return k.astype(np.float16), rng.standard_normal((B, H, n, D)).astype(np.float16)


@pytest.mark.parametrize("bits,G,R", [(2, 32, 64), (4, 32, 32), (2, 64, 128), (8, 32, 64)])
def test_streaming_equals_bulk(bits, G, R):
    """Appends (each followed by a key flush) give the same buffers as one
    bulk prefill of the same tokens with the same key window."""
    rng = np.random.default_rng(5 + bits + G + R)
    B, H, D, n = 2, 2, 128, 3 * R + 21
    cap = 4 * R
    k, v = _draw(rng, B, H, n, D)
    s = ovq.ValueQueueCache(B, H, D, bits, G, R, cap)
    for t in range(n):
        s.append(k[:, :, t], v[:, :, t])
        s.flush()
    assert s.status == 0
    bulk = ovq.ValueQueueCache(B, H, D, bits, G, R, cap)
    bulk.prefill(k, v, np.full(B, n), s.r_len.copy())
    assert bulk.status == 0
    for name in ("q_len", "r_len", "k_codes", "v_codes", "k_zero", "k_scale", "v_zero",
                 "v_scale", "v_res"):
        a, b = getattr(s, name), getattr(bulk, name)
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8)), name
    for b in range(B):   # the key window's live rows (the rest is stale)
        r = int(s.r_len[b])
        assert np.array_equal(s.k_res[b, :, :r].view(np.uint16), bulk.k_res[b, :, :r].view(np.uint16))


def test_evicted_values_have_the_bulk_per_token_codes():
    """The values that left the queue carry, token by token, the codes of
    the bulk per-token quantizer and of ``cache.value_queue``'s evictions;
    keys are those of the window-flush cache, bit for bit."""
    rng = np.random.default_rng(17)
    G, R, bits, D, n = 32, 64, 2, 128, 300
    k, v = _draw(rng, 1, 1, n, D)
    c = ovq.ValueQueueCache(1, 1, D, bits, G, R, 320)
    w = ocache.Cache(1, 1, D, bits, G, R, 320)
    for t in range(n):
        for x in (c, w):
            x.append(k[:, :, t], v[:, :, t])
            x.flush()
    vq = n - R
    evicted = ocache.value_queue(v[0, 0], R, G, bits)
    assert len(evicted) == vq
    st = c.head(0, 0)
    cv = ovq.unpack_tiles(st["v_codes"], bits)
    zv = ocache.untile_value_groups(st["v_zero"])
    sv = ocache.untile_value_groups(st["v_scale"])
    codes, zero, scale = oq.quantize_values(v[0, 0, :vq], G, bits)
    assert np.array_equal(cv[:vq], codes)
    assert np.array_equal(zv[:vq].view(np.uint16), zero.view(np.uint16))
    assert np.array_equal(sv[:vq].view(np.uint16), scale.view(np.uint16))
    for t, (ce, ze, se) in enumerate(evicted):
        assert np.array_equal(cv[t], ce) and np.array_equal(zv[t], ze) and np.array_equal(sv[t], se)
    assert not cv[vq:].any() and not zv[vq:].any()           # not yet quantized
    for name in ("k_codes", "k_zero", "k_scale", "q_len", "r_len"):
        assert np.array_equal(np.asarray(getattr(c, name)), np.asarray(getattr(w, name))), name


def test_hand_listed_token_layout():
    """T = 7 tokens, R = 4, G = 2: keys quantized for tokens 0..5 (the key
    window holds token 6), values quantized for tokens 0..2 (7 - 4) and fp16
    for 3..6, held in ring slots 3, 0, 1, 2.  The decode is the attention
    over exactly those rows."""
    rng = np.random.default_rng(3)
    D, G, R, bits = 4, 2, 4, 8
    k = rng.standard_normal((1, 1, 7, D)).astype(np.float16)
    v = rng.standard_normal((1, 1, 7, D)).astype(np.float16)
    c = ovq.ValueQueueCache(1, 1, D, bits, G, R, 8)
    c.prefill(k, v, np.array([7]))
    assert c.q_len[0] == 6 and c.r_len[0] == 1
    ring = c.v_res[0, 0]
    for t, slot in ((3, 3), (4, 0), (5, 1), (6, 2)):
        assert np.array_equal(ring[slot], v[0, 0, t])
    kq = oq.dequantize_keys(*oq.quantize_keys(k[0, 0, :6], G, bits), G)
    vq = oq.dequantize_values(*oq.quantize_values(v[0, 0, :3], G, bits), G)
    K = np.concatenate([kq, k[0, 0, 6:].astype(np.float64)])
    V = np.concatenate([vq, v[0, 0, 3:].astype(np.float64)])
    kk, vv = ovq.context(c.head(0, 0), G, bits, R)
    assert np.array_equal(kk, K) and np.array_equal(vv, V)
    q = rng.standard_normal(D).astype(np.float16)
    got = c.decode(q[None, None], 0.5)[0, 0]
    assert np.allclose(got, oatt.attention(q, K, V, 0.5), rtol=1e-13, atol=1e-15)


def test_queue_that_never_overflowed_keeps_every_value_in_fp16():
    """T <= R: no value has left the queue, so the decode is the attention
    over the quantized keys and the exact fp16 values."""
    rng = np.random.default_rng(9)
    D, G, R, bits, n = 128, 32, 128, 2, 100
    k, v = _draw(rng, 1, 1, n, D)
    c = ovq.ValueQueueCache(1, 1, D, bits, G, R, 256)
    c.prefill(k, v, np.array([n]))
    assert c.q_len[0] == 96 and not c.v_codes.any()
    kq = oq.dequantize_keys(*oq.quantize_keys(k[0, 0, :96], G, bits), G)
    K = np.concatenate([kq, k[0, 0, 96:].astype(np.float64)])
    q = (rng.standard_normal(D) / np.sqrt(D)).astype(np.float16)
    got = c.decode(q[None, None], 1.0)[0, 0]
    assert np.allclose(got, oatt.attention(q, K, v[0, 0].astype(np.float64), 1.0),
                       rtol=1e-13, atol=1e-15)


def test_bad_lengths_and_full_windows_are_flagged():
    rng = np.random.default_rng(4)
    k, v = _draw(rng, 2, 1, 80, 128)
    c = ovq.ValueQueueCache(2, 1, 128, 2, 32, 32, 64)
    c.prefill(k, v, np.array([70, 80]), np.array([6, 16]))   # 64 ok; 80 - 16 = 64 ok
    assert c.status == 0 and c.q_len.tolist() == [64, 64] and c.r_len.tolist() == [6, 16]
    c.prefill(k, v, np.array([70, 200]))                      # 200 > src_len
    assert c.status == ocache.ST_BAD_LENGTH
    c2 = ovq.ValueQueueCache(1, 1, 128, 2, 32, 32, 64)
    c2.prefill(k[:1], v[:1], np.array([64]), np.array([32]))  # full key window
    c2.append(k[:1, :, 0], v[:1, :, 0])
    assert c2.status == ocache.ST_RESIDUAL_FULL and c2.r_len[0] == 32
    c2.status = 0
    c2.flush()                                                # 32 + 32 <= 64
    assert c2.q_len[0] == 64 and c2.r_len[0] == 0 and c2.status == 0


# ------------------------------------------------------ planted mistakes

def _evict_newest(self, k_new, v_new):
    for b in range(self.batch):
        r = int(self.r_len[b])
        T = int(self.q_len[b]) + r
        slot = (T - 1) % self.R
        for h in range(self.heads):
            if T >= self.R:
                self._store_value(b, h, T - self.R, self.v_res[b, h, slot])
            self.v_res[b, h, T % self.R] = v_new[b, h]
            self.k_res[b, h, r] = k_new[b, h]
        self.r_len[b] = r + 1


def _one_more_quantized(t_total, residual):
    return max(0, int(t_total) - int(residual) + 1)


_FLUSH = ovq.ValueQueueCache.flush


def _flush_also_values(self):
    full = [int(r) == self.R for r in self.r_len]
    q0 = self.q_len.copy()
    _FLUSH(self)
    for b in range(self.batch):
        if full[b]:
            for h in range(self.heads):
                for t in range(self.R):
                    self._store_value(b, h, int(q0[b]) + t, self.v_res[b, h, t])


_CTX = ovq.context


def _ring_read_off_by_one(state, group, bits, residual):
    st = dict(state)
    st["v_res"] = np.roll(state["v_res"], 1, axis=0)
    return _CTX(st, group, bits, residual)


MUTANTS = [
    ("the newest value is evicted", ovq.ValueQueueCache, "append", _evict_newest),
    ("one value too many is quantized", ovq, "quantized_values", _one_more_quantized),
    ("the key flush also quantizes values", ovq.ValueQueueCache, "flush", _flush_also_values),
    ("the ring is read one slot off", ovq, "context", _ring_read_off_by_one),
]
PINS = [lambda: test_streaming_equals_bulk(2, 32, 64), test_evicted_values_have_the_bulk_per_token_codes,
        test_hand_listed_token_layout, test_queue_that_never_overflowed_keeps_every_value_in_fp16]


@pytest.mark.parametrize("label,owner,attr,mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(label, owner, attr, mutant, monkeypatch):
    monkeypatch.setattr(owner, attr, mutant)
    caught = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught, f"no pin caught: {label}"
