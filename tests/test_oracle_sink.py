"""CPU pins of the oracle's decode over an fp16 attention-sink segment
(unite.ai axis-selection guide, future-directions section: high-precision
windows for the recent and the attention-sink tokens)."""

import math

import numpy as np
import pytest

from oracle import cache as ocache
from oracle import rope as orope
from oracle import sink as osink
from oracle.attention import attention


def _textbook(q, k, v, alpha):
    """Softmax attention with plain loops (math.exp, fp64)."""
    D = len(q)
    scores = [alpha * sum(q[d] * row[d] for d in range(D)) for row in k]
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    return [sum(w[t] * v[t][d] for t in range(len(v))) / sum(w) for d in range(D)]


def _tiny(seed, S, bits, G, q_len=16, r_len=8, D=16, R=8):
    rng = np.random.default_rng(seed)
    n = q_len + r_len
    k = (rng.standard_normal((max(n, 1), D)) * 3).astype(np.float16)
    v = rng.standard_normal((max(n, 1), D)).astype(np.float16)
    sk = (rng.standard_normal((S, D)) * 3).astype(np.float16)
    sv = rng.standard_normal((S, D)).astype(np.float16)
    q = rng.standard_normal(D).astype(np.float16)
    st = ocache.head_state(k, v, q_len, r_len, G, bits, 32, R)
    return q, st, sk, sv


@pytest.mark.parametrize("bits,G,S", [(2, 4, 3), (4, 8, 1), (8, 4, 5)])
def test_sink_decode_matches_textbook_loops(bits, G, S):
    q, st, sk, sv = _tiny(70 + bits, S, bits, G)
    got = osink.decode_head_sink(q, st, sk, sv, 0.6, G, bits)
    kk, vv = ocache.context(st, G, bits)
    keys = sk.astype(np.float64).tolist() + kk.tolist()
    vals = sv.astype(np.float64).tolist() + vv.tolist()
    ref = _textbook(q.astype(np.float64).tolist(), keys, vals, 0.6)
    assert np.max(np.abs(got - np.array(ref))) <= 1e-12


def test_sink_tokens_count_as_window_tokens():
    """Without positions the sink may sit anywhere in the token set: the
    same rows placed at the end of the fp16 window give the same output."""
    rng = np.random.default_rng(80)
    D, G, R = 128, 32, 128
    k = (rng.standard_normal((200, D)) * 5).astype(np.float16)
    v = rng.standard_normal((200, D)).astype(np.float16)
    q = rng.standard_normal(D)
    S = 6
    sk, sv = k[160:160 + S], v[160:160 + S]
    st = ocache.head_state(k, v, 128, 32, G, 2, 256, R)
    got = osink.decode_head_sink(q, st, sk, sv, 0.05, G, 2)
    k2 = np.concatenate([k[:160], sk])
    v2 = np.concatenate([v[:160], sv])
    st2 = ocache.head_state(k2, v2, 128, 32 + S, G, 2, 256, R)
    ref = ocache.decode_head(q, st2, 0.05, G, 2)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_sink_alone_is_exact_fp16_attention():
    """An empty cache: attention over the fp16 sink rows as they are (no
    quantization touches them); one sink token gives its value row."""
    rng = np.random.default_rng(81)
    sk = (rng.standard_normal((9, 128)) * 4).astype(np.float16)
    sv = rng.standard_normal((9, 128)).astype(np.float16)
    q = rng.standard_normal(128)
    empty = ocache.head_state(sk[:1], sv[:1], 0, 0, 32, 2, 64, 32)
    got = osink.decode_head_sink(q, empty, sk, sv, 0.1, 32, 2)
    ref = _textbook(q.tolist(), sk.astype(np.float64).tolist(), sv.astype(np.float64).tolist(), 0.1)
    assert np.max(np.abs(got - np.array(ref))) <= 1e-12
    one = osink.decode_head_sink(q, empty, sk[:1], sv[:1], 0.1, 32, 2)
    assert np.array_equal(one, sv[0].astype(np.float64))


def test_one_sink_and_one_window_token_closed_form():
    """Two tokens: the output is sigma(alpha (q.k0 - q.k1)) v0 + (1 - sigma) v1."""
    def row(*x):   # 16 channels, the rest 0
        return np.pad(np.array(x, np.float64), (0, 16 - len(x)))
    q = row(1.0, -2.0, 0.5, 0.0)
    k0 = row(2.0, 0.0, 1.0, 3.0).astype(np.float16)[None]
    v0 = row(1.0, 2.0, 3.0, 4.0, -5.0).astype(np.float16)[None]
    k1 = row(0.0, 1.0, 0.0, -1.0).astype(np.float16)[None]
    v1 = row(-1.0, 0.5, 0.25, 8.0, 0.0, 6.0).astype(np.float16)[None]
    st = ocache.head_state(k1, v1, 0, 1, 4, 2, 4, 4)
    alpha = 0.75
    got = osink.decode_head_sink(q, st, k0, v0, alpha, 4, 2)
    s0, s1 = alpha * 2.5, alpha * -2.0   # q.k0 = 2 + 0.5, q.k1 = -2
    sig = 1.0 / (1.0 + math.exp(s1 - s0))
    ref = sig * v0[0].astype(np.float64) + (1 - sig) * v1[0].astype(np.float64)
    assert np.max(np.abs(got - ref)) <= 1e-15


def test_no_sink_is_the_plain_decode():
    q, st, sk, sv = _tiny(82, 0, 2, 4)
    assert np.array_equal(osink.decode_head_sink(q, st, sk, sv, 0.6, 4, 2),
                          ocache.decode_head(q, st, 0.6, 4, 2))


# ------------------------------------------------ with the rotary embedding

def test_rotary_sink_is_the_start_of_a_window_only_cache():
    """A cache with no quantized tokens: n_sink sink rows then r window rows
    at positions 0 .. n_sink + r - 1 are a window-only cache holding both
    (the rotary oracle's decode, pinned on its own)."""
    rng = np.random.default_rng(83)
    D, S, r = 128, 7, 20
    k = (rng.standard_normal((S + r, D)) * 4).astype(np.float16)
    v = rng.standard_normal((S + r, D)).astype(np.float16)
    q = rng.standard_normal(D)
    st = ocache.head_state(k[S:], v[S:], 0, r, 32, 2, 64, 32)
    got = osink.decode_head_sink(q, st, k[:S], v[:S], 0.1, 32, 2, rope_base=10000.0)
    both = ocache.head_state(k, v, 0, S + r, 32, 2, 64, 32)
    ref = orope.decode_head_rope(q, both, 0.1, 32, 2, 10000.0)
    assert np.max(np.abs(got - ref)) <= 1e-12


@pytest.mark.parametrize("bits,G,S", [(2, 4, 3), (4, 8, 2)])
def test_rotary_sink_decode_matches_textbook_loops(bits, G, S):
    """Quantized tokens after the sink sit at positions S, S + 1, ...:
    loops over tokens and channel pairs with math.cos / math.sin."""
    q, st, sk, sv = _tiny(90 + bits, S, bits, G)
    got = osink.decode_head_sink(q, st, sk, sv, 0.6, G, bits, rope_base=50.0)
    kk, vv = ocache.context(st, G, bits)
    keys = sk.astype(np.float64).tolist() + kk.tolist()
    vals = sv.astype(np.float64).tolist() + vv.tolist()
    D, base = len(q), 50.0
    rot = []
    for t, row in enumerate(keys):
        y = list(row)
        for f in range(D // 2):
            th = t * base ** (-2.0 * f / D)
            a, b = row[2 * f], row[2 * f + 1]
            y[2 * f] = a * math.cos(th) - b * math.sin(th)
            y[2 * f + 1] = a * math.sin(th) + b * math.cos(th)
        rot.append(y)
    ref = _textbook(q.astype(np.float64).tolist(), rot, vals, 0.6)
    assert np.max(np.abs(got - np.array(ref))) <= 1e-12


def test_rotary_without_sink_is_the_rotary_decode():
    q, st, sk, sv = _tiny(84, 0, 2, 4)
    assert np.array_equal(osink.decode_head_sink(q, st, sk, sv, 0.6, 4, 2, rope_base=50.0),
                          orope.decode_head_rope(q, st, 0.6, 4, 2, 50.0))


# ------------------------------------------------------------ planted mistakes
# Each mutant replaces the oracle's sink decode with a plausible slip; at
# least one pin above must fail with it in place.

def _mutant(kind):
    def f(q, state, sink_k, sink_v, alpha, group, bits, rope_base=None):
        kk, vv = ocache.context(state, group, bits)
        sk = np.asarray(sink_k, np.float64).reshape(-1, kk.shape[1])
        sv = np.asarray(sink_v, np.float64).reshape(-1, vv.shape[1])
        if kind == "dropped":
            sk, sv = sk[:0], sv[:0]
        elif kind == "twice":
            sk, sv = np.concatenate([sk, sk]), np.concatenate([sv, sv])
        elif kind == "swapped":
            sk, sv = sv, sk
        elif kind == "shifted":      # sink values paired with the next key
            sv = np.roll(sv, 1, axis=0)
        elif kind == "unscaled":     # sink scores without alpha
            sk = sk / alpha
        if rope_base is not None:
            if kind == "cache_from_zero":    # cache positions not moved past the sink
                return attention(q, np.concatenate([orope.rope(sk, np.arange(len(sk)), rope_base),
                                                    orope.rope(kk, np.arange(len(kk)), rope_base)]),
                                 np.concatenate([sv, vv]), alpha)
            if kind == "sink_unrotated":
                return attention(q, np.concatenate([sk, orope.rope(kk, np.arange(len(kk)) + len(sk),
                                                                   rope_base)]),
                                 np.concatenate([sv, vv]), alpha)
            keys = orope.rope(np.concatenate([sk, kk]), np.arange(len(sk) + len(kk)), rope_base)
            return attention(q, keys, np.concatenate([sv, vv]), alpha)
        return attention(q, np.concatenate([sk, kk]), np.concatenate([sv, vv]), alpha)
    return f


PINS = [lambda: test_sink_decode_matches_textbook_loops(2, 4, 3),
        test_sink_tokens_count_as_window_tokens, test_sink_alone_is_exact_fp16_attention,
        test_one_sink_and_one_window_token_closed_form,
        test_rotary_sink_is_the_start_of_a_window_only_cache,
        lambda: test_rotary_sink_decode_matches_textbook_loops(2, 4, 3)]


@pytest.mark.parametrize("kind", ["dropped", "twice", "swapped", "shifted", "unscaled",
                                  "cache_from_zero", "sink_unrotated"])
def test_planted_mistake_is_caught(kind, monkeypatch):
    monkeypatch.setattr(osink, "decode_head_sink", _mutant(kind))
    caught = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0
