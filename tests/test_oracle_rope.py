"""CPU pins of the oracle's rotary embedding and pre-rotation-key decode
(unite.ai axis-selection guide, rotary-embedding section: keys quantized
before the rotation, rotated after dequantization)."""

import cmath
import math

import numpy as np
import pytest

from oracle import cache as ocache
from oracle import rope as orope


def test_position_zero_is_the_identity():
    x = np.random.default_rng(1).standard_normal((3, 128))
    assert np.array_equal(orope.rope(x, [0, 0, 0], 10000.0), x)


def test_rotation_direction_and_pairing_match_complex_multiplication():
    """Pair f = (2f, 2f+1) read as the complex number x[2f] + i x[2f+1] is
    multiplied by exp(i p theta_f): counter-clockwise, adjacent channels."""
    # D = 2: theta_0 = 1, so (1, 0) at position p becomes (cos p, sin p)
    for p in (1, 2, 7, 1000):
        y = orope.rope(np.array([[1.0, 0.0]]), [p], 10000.0)[0]
        z = cmath.exp(1j * p)
        assert abs(y[0] - z.real) < 1e-12 and abs(y[1] - z.imag) < 1e-12
    # D = 4, base 10000: theta_1 = 10000^(-1/2) = 0.01, so at p = 100 the
    # second pair turns by exactly 1 radian and the first by 100
    y = orope.rope(np.array([[0.0, 0.0, 2.0, -3.0]]), [100], 10000.0)[0]
    z1 = complex(2.0, -3.0) * cmath.exp(1j * 1.0)
    assert abs(y[2] - z1.real) < 1e-12 and abs(y[3] - z1.imag) < 1e-12
    assert y[0] == 0.0 and y[1] == 0.0
    y = orope.rope(np.array([[0.5, 1.5, 0.0, 0.0]]), [100], 10000.0)[0]
    z0 = complex(0.5, 1.5) * cmath.exp(1j * 100.0)
    assert abs(y[0] - z0.real) < 1e-12 and abs(y[1] - z0.imag) < 1e-12


def test_norm_is_preserved():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 128)) * 30
    pos = rng.integers(0, 131072, 50)
    y = orope.rope(x, pos, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 128))
    k = rng.standard_normal((1, 128))
    for m, n, s in [(5, 9, 100), (0, 4000, 127000), (130000, 3, 1)]:
        a = orope.rope(q, [m], 10000.0) @ orope.rope(k, [n], 10000.0).T
        b = orope.rope(q, [m + s], 10000.0) @ orope.rope(k, [n + s], 10000.0).T
        assert abs(a - b).max() <= 1e-9 * (1 + abs(a).max())


def test_rotations_compose():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4, 16))
    a, b = np.array([3, 50, 1000, 0]), np.array([7, 1, 20000, 5])
    np.testing.assert_allclose(orope.rope(orope.rope(x, a, 500.0), b, 500.0),
                               orope.rope(x, a + b, 500.0), atol=1e-11)


def _textbook_rope_decode(q, k, v, alpha, base):
    """Loops over tokens and channel pairs with math.cos / math.sin."""
    D = len(q)
    scores = []
    for t, row in enumerate(k):
        s = 0.0
        for f in range(D // 2):
            th = t * base ** (-2.0 * f / D)
            a, b = row[2 * f], row[2 * f + 1]
            s += q[2 * f] * (a * math.cos(th) - b * math.sin(th))
            s += q[2 * f + 1] * (a * math.sin(th) + b * math.cos(th))
        scores.append(alpha * s)
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    return [sum(w[t] * v[t][d] for t in range(len(v))) / sum(w) for d in range(D)]


@pytest.mark.parametrize("bits,G", [(2, 4), (4, 8), (8, 4)])
def test_rope_decode_matches_textbook_loops(bits, G):
    rng = np.random.default_rng(60 + bits)
    D, R, L = 16, 8, 24          # 16 quantized tokens + 8 window tokens
    k = (rng.standard_normal((L + R, D)) * 3).astype(np.float16)
    v = rng.standard_normal((L + R, D)).astype(np.float16)
    q = rng.standard_normal(D).astype(np.float16)
    st = ocache.head_state(k, v, 16, 8, G, bits, 32, R)
    got = orope.decode_head_rope(q, st, 0.7, G, bits, 50.0)
    kk, vv = ocache.context(st, G, bits)
    ref = _textbook_rope_decode(q.astype(np.float64).tolist(), kk.tolist(), vv.tolist(), 0.7, 50.0)
    assert np.max(np.abs(got - np.array(ref))) <= 1e-12


def test_rope_decode_of_one_token_is_its_value_row():
    rng = np.random.default_rng(7)
    k = rng.standard_normal((1, 128)).astype(np.float16)
    v = rng.standard_normal((1, 128)).astype(np.float16)
    st = ocache.head_state(k, v, 0, 1, 32, 2, 32, 32)
    out = orope.decode_head_rope(rng.standard_normal(128), st, 1.0, 32, 2, 10000.0)
    assert np.array_equal(out, v[0].astype(np.float64))


def test_rope_decode_differs_from_plain_decode():
    """The rotation matters: with a spread-out softmax the outputs differ,
    and at position 0 alone (a one-token cache) they agree."""
    rng = np.random.default_rng(8)
    k = (rng.standard_normal((64, 128)) * 3).astype(np.float16)
    v = rng.standard_normal((64, 128)).astype(np.float16)
    q = rng.standard_normal(128)
    st = ocache.head_state(k, v, 32, 32, 32, 2, 64, 32)
    a = orope.decode_head_rope(q, st, 0.02, 32, 2, 10000.0)
    b = ocache.decode_head(q, st, 0.02, 32, 2)
    assert np.abs(a - b).max() > 1e-2
    st1 = ocache.head_state(k[:1], v[:1], 0, 1, 32, 2, 64, 32)
    assert np.array_equal(orope.decode_head_rope(q, st1, 0.02, 32, 2, 10000.0),
                          ocache.decode_head(q, st1, 0.02, 32, 2))


# ------------------------------------------------------------ planted mistakes
# Each mutant replaces the oracle's rotation (or its decode) with a plausible
# slip; at least one of the pins above must fail with it in place.

def _rope_generic(x, positions, base, sign=1.0, half=False, expo=2.0, shift=0):
    x = np.asarray(x, dtype=np.float64)
    T, D = x.shape
    f = np.arange(D // 2, dtype=np.float64)
    th = np.float64(base) ** (-expo * f / D)
    ang = (np.asarray(positions, dtype=np.float64)[:, None] + shift) * th[None, :]
    c, s = np.cos(ang), sign * np.sin(ang)
    ia, ib = (np.arange(D // 2), np.arange(D // 2) + D // 2) if half else \
        (np.arange(0, D, 2), np.arange(1, D, 2))
    a, b = x[:, ia], x[:, ib]
    y = np.empty_like(x)
    y[:, ia] = a * c - b * s
    y[:, ib] = a * s + b * c
    return y


def _decode_window_restarts(q, state, alpha, group, bits, base):
    kk, vv = ocache.context(state, group, bits)
    ql = state["q_len"]
    pos = np.concatenate([np.arange(ql), np.arange(kk.shape[0] - ql)])
    return orope.attention(q, orope.rope(kk, pos, base), vv, alpha)


_ROPE_PINS = [test_position_zero_is_the_identity,
              test_rotation_direction_and_pairing_match_complex_multiplication,
              test_norm_is_preserved, test_scores_depend_on_relative_position_only,
              test_rotations_compose, test_rope_decode_of_one_token_is_its_value_row,
              test_rope_decode_differs_from_plain_decode]


@pytest.mark.parametrize("label,attr,mutant", [
    ("clockwise rotation", "rope", lambda x, p, b: _rope_generic(x, p, b, sign=-1.0)),
    ("rotate-half pairing", "rope", lambda x, p, b: _rope_generic(x, p, b, half=True)),
    ("frequency exponent f/D", "rope", lambda x, p, b: _rope_generic(x, p, b, expo=1.0)),
    ("positions off by one", "rope", lambda x, p, b: _rope_generic(x, p, b, shift=1)),
    ("window positions restart at 0", "decode_head_rope", _decode_window_restarts),
])
def test_rope_pins_catch_planted_mistake(label, attr, mutant, monkeypatch):
    monkeypatch.setattr(orope, attr, mutant)
    caught = []
    for pin in _ROPE_PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    for bits, G in [(2, 4), (4, 8)]:
        try:
            test_rope_decode_matches_textbook_loops(bits, G)
        except AssertionError:
            caught.append("textbook")
    assert caught, f"no pin caught: {label}"
