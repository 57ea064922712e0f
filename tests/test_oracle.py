"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test ties one oracle function to something other than itself: hand-worked
cases, exact brute force, closed forms, or invariants of the definitions.
The page references are:
  * unite.ai axis-selection guide -- quantization-error section (min as
    zero-point, step = range / (2^B - 1), round to nearest, error <= step/2),
    keys section (per-channel key groups), values section (per-token value
    groups; output = softmax-weighted sum of values), systems section (fp16
    window of recent tokens, quantized once enough accumulate).
  * discosf KIVI tutorial -- section 2.1 (cache-size formula), section 3.1
    (groups of G tokens plus a remainder window), section 3.2 (value queue).
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import cache as ocache
from oracle import packing as opack
from oracle import quantizer as oq
from bit_kv_cache_decode_amd import workloads as wl

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _read_cases(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([p.strip() for p in line.split(";")])
    return rows


# ----------------------------------------------------------------- quantizer

def test_quantizer_hand_cases(golden_dir):
    rows = _read_cases(os.path.join(golden_dir, "quantizer_cases.txt"))
    assert len(rows) >= 10
    for bits, xs, codes, zero, scale, _why in rows:
        x = np.array([float(t) for t in xs.split()], dtype=np.float16)
        c, z, s = oq.quantize_groups(x[None, :], int(bits))
        assert c[0].tolist() == [int(t) for t in codes.split()], (xs, c)
        # compare fp16 bit patterns, so a -0 zero-point would fail against "0"
        assert z[0].view(np.uint16) == np.float16(float(zero)).view(np.uint16), (xs, z)
        assert s[0].view(np.uint16) == np.float16(float(scale)).view(np.uint16), (xs, s)


def _exact_nearest(x, mn, s, bits):
    """Nearest level mn + k*s over k in [0, 2^B-1], exact rationals, ties to
    the even k.  Returns (k, distance of the exact quotient to a half-integer)."""
    if s == 0:
        return 0, Fraction(1)
    X, M, S = Fraction(float(x)), Fraction(float(mn)), Fraction(float(s))
    best = None
    for k in range(2 ** bits):
        d = abs(X - (M + k * S))
        if best is None or d < best[1] or (d == best[1] and k % 2 == 0):
            best = (k, d)
    quo = (X - M) / S
    tie_gap = abs(quo - (math.floor(quo) + Fraction(1, 2)))
    return best[0], tie_gap


@pytest.mark.parametrize("bits,n_groups", [(2, 400), (4, 400), (8, 60)])
def test_quantizer_matches_exact_brute_force(bits, n_groups):
    rng = np.random.default_rng(7 + bits)
    n = 16
    scale = rng.choice([1e-3, 1.0, 30.0, 300.0], size=(n_groups, 1))
    x = (rng.standard_normal((n_groups, n)) * scale).astype(np.float16)
    x[::7, 3] *= np.float16(40.0)                       # outliers inside groups
    codes, zero, step = oq.quantize_groups(x, bits)
    near_ties = 0
    for g in range(n_groups):
        for i in range(n):
            k, gap = _exact_nearest(x[g, i], zero[g], step[g], bits)
            if gap < Fraction(1, 2 ** 18):
                near_ties += 1                          # fp32 quotient rounding may decide
                continue
            assert codes[g, i] == k, (g, i, x[g], codes[g], k)
    assert near_ties < n_groups * n // 100


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_error_at_most_half_step(bits):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((2000, 32)) * rng.choice([0.01, 1, 50], (2000, 1))).astype(np.float16)
    codes, zero, step = oq.quantize_groups(x, bits)
    normal = step.astype(np.float64) >= 2.0 ** -14      # exclude fp16-subnormal steps
    xhat = zero.astype(np.float64)[:, None] + codes * step.astype(np.float64)[:, None]
    err = np.abs(xhat - x.astype(np.float64))
    bound = step.astype(np.float64)[:, None] / 2 * (1 + 2.0 ** -20)
    assert np.all(err[normal] <= bound[normal])
    assert normal.mean() > 0.99


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_min_maps_to_zero_and_max_to_top_code(bits):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((500, 32)).astype(np.float16)
    codes, zero, step = oq.quantize_groups(x, bits)
    rows = np.arange(500)
    assert np.all(codes[rows, x.argmin(1)] == 0)
    assert np.all(codes[rows, x.argmax(1)] == 2 ** bits - 1)
    assert np.all(zero == x.min(1))
    assert codes.max() <= 2 ** bits - 1


def test_constant_groups_reconstruct_exactly():
    x = np.repeat(np.array([[-3.5], [0.0], [7.25], [65504.0]], np.float16), 32, axis=1)
    for bits in (2, 4, 8):
        codes, zero, step = oq.quantize_groups(x, bits)
        assert np.all(codes == 0) and np.all(step == 0)
        xhat = oq.dequantize_values(codes, zero[:, None], step[:, None], 32)
        assert np.array_equal(xhat, x.astype(np.float64))


def test_step_formula_is_range_over_levels():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((300, 32)).astype(np.float16)
    for bits in (2, 4, 8):
        _, _, step = oq.quantize_groups(x, bits)
        rngv = x.max(1).astype(np.float64) - x.min(1).astype(np.float64)
        # fp16 step within half an fp16 ulp (plus fp32 rounding) of range / (2^B - 1)
        rel = np.abs(step.astype(np.float64) - rngv / (2 ** bits - 1)) / (rngv / (2 ** bits - 1))
        assert rel.max() <= 2.0 ** -11 * (1 + 2.0 ** -10)


def test_dequantization_is_exact():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((64, 128)).astype(np.float16)
    codes, zero, step = oq.quantize_values(x, 32, 2)
    xhat = oq.dequantize_values(codes, zero, step, 32)
    for t, d in [(0, 0), (5, 77), (63, 127), (17, 31)]:
        exact = Fraction(float(zero[t, d // 32])) + int(codes[t, d]) * Fraction(float(step[t, d // 32]))
        assert Fraction(xhat[t, d]) == exact
    ck, zk, sk = oq.quantize_keys(x, 32, 2)
    khat = oq.dequantize_keys(ck, zk, sk, 32)
    for t, d in [(0, 0), (5, 77), (63, 127), (40, 31)]:
        exact = Fraction(float(zk[t // 32, d])) + int(ck[t, d]) * Fraction(float(sk[t // 32, d]))
        assert Fraction(khat[t, d]) == exact
    # the reconstruction of both axes stays within half a step of the input
    assert np.all(np.abs(khat - x) <= np.repeat(sk.astype(np.float64), 32, 0) / 2 * (1 + 2.0 ** -20))


def test_key_and_value_axes_are_transposes():
    """A key tile [G, D] quantized per channel equals the transposed tile
    [D, G] quantized per token with group G (one group per row)."""
    rng = np.random.default_rng(21)
    for G, bits in [(32, 2), (128, 2), (32, 4), (64, 4), (32, 8), (128, 8)]:
        tile = rng.standard_normal((G, 128)).astype(np.float16)
        tile[:, 5] *= np.float16(60)
        ck, zk, sk = oq.quantize_keys(tile, G, bits)
        cv, zv, sv = oq.quantize_values(np.ascontiguousarray(tile.T), G, bits)
        assert np.array_equal(ck, cv.T)
        assert np.array_equal(zk[0], zv[:, 0]) and np.array_equal(sk[0], sv[:, 0])


def test_key_groups_are_per_channel_over_tokens():
    """An outlier channel only inflates its own key groups, and an outlier
    token only inflates its own value groups (keys/values sections)."""
    rng = np.random.default_rng(4)
    k = rng.standard_normal((64, 128)).astype(np.float16)
    base = oq.quantize_keys(k, 32, 2)
    k2 = k.copy()
    k2[:, 9] *= np.float16(80)
    out = oq.quantize_keys(k2, 32, 2)
    changed = np.argwhere(out[2] != base[2])
    assert set(changed[:, 1].tolist()) == {9}
    v2 = k.copy()
    v2[40] *= np.float16(80)
    vb, vo = oq.quantize_values(k, 32, 2), oq.quantize_values(v2, 32, 2)
    assert set(np.argwhere(vo[2] != vb[2])[:, 0].tolist()) == {40}


# ------------------------------------------------------------------- packing

def test_packing_hand_cases(golden_dir):
    for bits, G, D, toks, words in _read_cases(os.path.join(golden_dir, "packing_cases.txt")):
        bits, G, D = int(bits), int(G), int(D)
        codes = np.array([[int(c) for c in t.split()] for t in toks.split("|")], np.uint8)
        assert codes.shape == (G, D)
        packed = opack.pack_tiles(codes, G, bits)
        assert [int(w) for w in packed.reshape(-1)] == [int(w, 16) for w in words.split()]
        assert np.array_equal(opack.unpack_tiles(packed, bits), codes)


def test_value_group_tile_order_hand_cases(golden_dir):
    """Value zero-points and steps land in the documented tile order
    [n / G][j][n % G] (hand-worked fixtures), and dequantizing a cache that
    holds those tiles gives the rows back exactly (every value of the
    fixtures is on a level of its group)."""
    rows = _read_cases(os.path.join(golden_dir, "value_tile_cases.txt"))
    assert len(rows) >= 2
    for bits, G, D, toks, zeros, steps, _why in rows:
        bits, G, D = int(bits), int(G), int(D)
        v = np.array([[float(x) for x in t.split()] for t in toks.split("|")], np.float16)
        assert v.shape[1] == D and v.shape[0] % G == 0
        enc = ocache.encode_tokens(v, v, G, bits)
        assert enc["v_zero"].shape == (v.shape[0] // G, D // G, G)
        assert enc["v_zero"].reshape(-1).tolist() == [float(x) for x in zeros.split()]
        assert enc["v_scale"].reshape(-1).tolist() == [float(x) for x in steps.split()]
        st = ocache.head_state(v, v, v.shape[0], 0, G, bits, v.shape[0], G)
        _, vv = ocache.context(st, G, bits)
        assert np.array_equal(vv, v.astype(np.float64))


@pytest.mark.parametrize("bits,G", [(2, 32), (2, 128), (4, 32), (4, 128), (8, 32), (8, 128)])
def test_pack_unpack_round_trip(bits, G):
    rng = np.random.default_rng(bits * G)
    codes = rng.integers(0, 2 ** bits, size=(2 * G, 128), dtype=np.uint8)
    packed = opack.pack_tiles(codes, G, bits)
    assert packed.shape == (2, 128 * bits // 32, G) and packed.dtype == np.uint32
    assert np.array_equal(opack.unpack_tiles(packed, bits), codes)


# ----------------------------------------------------------------- streaming

def _small_kv(rng, n, D=128, outlier=True):
    k = rng.standard_normal((n, D)).astype(np.float32)
    if outlier:
        k[:, 17] *= 40
    return k.astype(np.float16), rng.standard_normal((n, D)).astype(np.float16)


@pytest.mark.parametrize("bits,G,R", [(2, 32, 128), (2, 32, 32), (4, 128, 128), (2, 64, 128), (8, 32, 64)])
def test_streaming_equals_bulk(bits, G, R):
    """Token-by-token appends with flushes at R give the same buffers as one
    bulk prefill of the same tokens (tutorial section 3.1 streaming rule)."""
    rng = np.random.default_rng(31)
    batch, heads, n, cap = 2, 2, 3 * R + 37, 4 * R
    k = rng.standard_normal((batch, heads, n, 128)).astype(np.float16)
    v = rng.standard_normal((batch, heads, n, 128)).astype(np.float16)
    s = ocache.Cache(batch, heads, 128, bits, G, R, cap)
    for t in range(n):
        s.append(k[:, :, t], v[:, :, t])
        s.flush()
    b = ocache.Cache(batch, heads, 128, bits, G, R, cap)
    b.prefill(k, v, np.full(batch, n), np.full(batch, n % R))
    assert s.status == 0 and b.status == 0
    assert np.array_equal(s.q_len, b.q_len) and np.array_equal(s.r_len, b.r_len)
    for name in ("k_codes", "v_codes", "k_zero", "k_scale", "v_zero", "v_scale"):
        assert np.array_equal(getattr(s, name), getattr(b, name)), name
    r = n % R
    assert np.array_equal(s.k_res[:, :, :r], b.k_res[:, :, :r])


def test_value_queue_variant_gives_same_codes():
    """The value queue of tutorial section 3.2 (pop the oldest token once R
    are queued, quantize it per token) encodes every token exactly as the
    bulk per-token quantizer does: per-token groups carry no state."""
    rng = np.random.default_rng(8)
    _, v = _small_kv(rng, 300)
    evicted = ocache.value_queue(v, residual=64, group=32, bits=2)
    assert len(evicted) == 300 - 64
    codes, zero, step = oq.quantize_values(v, 32, 2)
    for t, (c, z, s) in enumerate(evicted):
        assert np.array_equal(c, codes[t]) and np.array_equal(z, zero[t]) and np.array_equal(s, step[t])


def test_prefill_default_remainder_and_status_bits():
    rng = np.random.default_rng(12)
    k = rng.standard_normal((3, 1, 300, 128)).astype(np.float16)
    c = ocache.Cache(3, 1, 128, 2, 32, 64, 256)
    c.prefill(k, k, np.array([100, 300, 64]))
    # 100 = 3*32 + 4 -> 96 quantized + 4 window; 300 -> 288 > capacity 256;
    # 64 -> 64 + 0
    assert c.q_len.tolist() == [96, 0, 64] and c.r_len.tolist() == [4, 0, 0]
    assert c.status == ocache.ST_CAPACITY
    c2 = ocache.Cache(1, 1, 128, 2, 32, 64, 256)
    c2.prefill(k[:1], k[:1], np.array([100]), np.array([5]))          # 95 not a multiple of 32
    assert c2.status == ocache.ST_BAD_LENGTH and c2.q_len[0] == 0
    c3 = ocache.Cache(1, 1, 128, 2, 32, 32, 256)
    c3.prefill(k[:1], k[:1], np.array([64]), np.array([32]))
    c3.append(k[:1, :, 0], k[:1, :, 0])
    assert c3.status == ocache.ST_RESIDUAL_FULL and c3.r_len[0] == 32


# ----------------------------------------------------------------- attention

def _textbook(q, K, V, alpha):
    """Pure-Python softmax attention: loops and math.exp, no numpy."""
    T, D = len(K), len(q)
    if T == 0:
        return [0.0] * D
    s = [alpha * math.fsum(float(q[d]) * float(K[t][d]) for d in range(D)) for t in range(T)]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    z = math.fsum(w)
    return [math.fsum(w[t] * float(V[t][d]) for t in range(T)) / z for d in range(D)]


def test_attention_closed_form():
    # scores 0 and ln 3 -> weights 1/4, 3/4 -> output 1/4 * 1 + 3/4 * 5 = 4
    out = oatt.attention(np.array([1.0]), np.array([[0.0], [1.0]]), np.array([[1.0], [5.0]]), math.log(3.0))
    assert abs(out[0] - 4.0) < 1e-15


@pytest.mark.parametrize("bits,G", [(2, 4), (4, 8), (2, 8), (8, 4)])
def test_attention_matches_textbook_loops(bits, G):
    rng = np.random.default_rng(40 + bits + G)
    D, L = 16, 48
    k = (rng.standard_normal((L, D)) * 3).astype(np.float16)
    v = rng.standard_normal((L, D)).astype(np.float16)
    q = rng.standard_normal(D).astype(np.float16)
    ck, zk, sk = oq.quantize_keys(k, G, bits)
    cv, zv, sv = oq.quantize_values(v, G, bits)
    K = oq.dequantize_keys(ck, zk, sk, G)
    V = oq.dequantize_values(cv, zv, sv, G)
    ref = _textbook(q, K.tolist(), V.tolist(), 0.7)
    assert np.max(np.abs(oatt.attention(q, K, V, 0.7) - np.array(ref))) <= 1e-12


def test_residual_only_cache_is_exact_fp16_attention():
    rng = np.random.default_rng(2)
    k, v = _small_kv(rng, 40)
    q = (rng.standard_normal(128) / math.sqrt(128)).astype(np.float16)
    st = ocache.head_state(k, v, 0, 40, 32, 2, 64, 64)
    out = ocache.decode_head(q, st, 1.0, 32, 2)
    ref = _textbook(q, k.astype(np.float64).tolist(), v.astype(np.float64).tolist(), 1.0)
    assert np.max(np.abs(out - np.array(ref))) <= 1e-12


def test_zero_query_gives_mean_of_dequantized_values():
    rng = np.random.default_rng(13)
    k, v = _small_kv(rng, 160)
    st = ocache.head_state(k, v, 128, 32, 32, 2, 256, 128)
    K, V = ocache.context(st, 32, 2)
    out = ocache.decode_head(np.zeros(128, np.float16), st, 1.0, 32, 2)
    assert np.max(np.abs(out - V.mean(0))) <= 1e-12
    assert K.shape == (160, 128)


def test_single_token_context_returns_its_value_row():
    rng = np.random.default_rng(14)
    k, v = _small_kv(rng, 1)
    st = ocache.head_state(k, v, 0, 1, 32, 2, 64, 64)
    q = rng.standard_normal(128).astype(np.float16)
    assert np.array_equal(ocache.decode_head(q, st, 1.0, 32, 2), v[0].astype(np.float64))


def test_empty_context_gives_zero():
    st = ocache.head_state(np.zeros((0, 128), np.float16), np.zeros((0, 128), np.float16),
                           0, 0, 32, 2, 64, 64)
    assert np.all(ocache.decode_head(np.ones(128, np.float16), st, 1.0, 32, 2) == 0)


def test_token_permutation_invariance():
    rng = np.random.default_rng(15)
    k, v = _small_kv(rng, 96)
    st = ocache.head_state(k, v, 64, 32, 32, 2, 128, 64)
    K, V = ocache.context(st, 32, 2)
    q = (rng.standard_normal(128) / 11).astype(np.float16)
    perm = rng.permutation(K.shape[0])
    a = oatt.attention(q, K, V, 1.0)
    b = oatt.attention(q, K[perm], V[perm], 1.0)
    assert np.max(np.abs(a - b)) <= 1e-12


def test_split_merge_equals_single_pass():
    rng = np.random.default_rng(16)
    k, v = _small_kv(rng, 500)
    q = (rng.standard_normal(128) / 11).astype(np.float16)
    K, V = k.astype(np.float64), v.astype(np.float64)
    full = oatt.attention(q, K, V, 1.0)
    for cuts in ([250], [1, 2, 3, 499], [100, 200, 300, 400], [0, 0, 500]):
        edges = [0] + cuts + [500]
        parts = [oatt.partial(q, K[a:b], V[a:b], 1.0) for a, b in zip(edges[:-1], edges[1:])]
        assert np.max(np.abs(oatt.merge(parts) - full)) <= 1e-12


# ---------------------------------------------------------------- byte model

def test_fp16_byte_model_matches_stated_sizes(golden_dir):
    for name, b, s, layers, hidden, stated, tol, _src in _read_cases(os.path.join(golden_dir, "byte_model.txt")):
        got = wl.fp16_kv_cache_bytes(int(b), int(s), int(layers), int(hidden))
        assert abs(got - float(stated)) <= float(tol) * float(stated), name
    # tutorial section 1: 10 GB free holds about 20,000 tokens of LLaMA2-7B
    assert 19000 < (10 * 2 ** 30) // wl.fp16_kv_cache_bytes(1, 1, 32, 4096) < 21000


def test_decode_byte_model_per_head():
    # 3968 quantized + 128 window tokens, D=128, B=2, G=32:
    # codes 2*3968*32 + K meta 124*128*4 + V meta 3968*4*4 + window 2*128*256 + q 256 + out 512
    assert wl.decode_bytes_per_head(3968, 128, 128, 2, 32) == 447232
    assert wl.decode_bytes_per_head(0, 0, 128, 2, 32) == 768


def test_step_byte_model():
    # the Llama-2-7B-shaped layer, every window filled by the step's append:
    # decode bytes + new K/V rows (2*128*2 per head) + flush writes per head
    # (codes 2*128*128*2/8, K meta 4*128*4, V meta 128*4*4)
    ql = np.full(8, 3968)
    assert wl.step_bytes(ql, np.full(8, 127), 32, 128, 2, 32, 128) == \
        256 * (447232 + 512 + 8192 + 2048 + 2048)
    # a window the append does not fill: no flush bytes
    assert wl.step_bytes(ql[:1], np.array([5]), 1, 128, 2, 32, 128) == \
        wl.decode_bytes_per_head(3968, 6, 128, 2, 32) + 512


# ----------------------------------------------------------------- direction

def test_per_channel_keys_beat_per_token_keys_on_outlier_channels():
    """Keys section: outliers that sit in fixed channels spoil every per-token
    key group but only their own per-channel groups, so per-channel grouping
    gives lower reconstruction error on the workload keys, and lower
    reconstruction and score error when the outlier channels carry a
    persistent large magnitude on every token (direction only: the page's
    figures need real activations)."""
    w = wl.generate(2, batch=1)
    k = w.k[0, 0, :1024]
    kf = k.astype(np.float64)

    def both(keys):
        ck, zk, sk = oq.quantize_keys(keys, 32, 2)
        ct, zt, st = oq.quantize_values(keys, 32, 2)     # per-token grouping of keys
        return oq.dequantize_keys(ck, zk, sk, 32), oq.dequantize_values(ct, zt, st, 32)

    per_channel, per_token = both(k)
    assert np.abs(per_channel - kf).mean() < np.abs(per_token - kf).mean()

    rng = np.random.default_rng(17)
    keys = rng.standard_normal((1024, 128)).astype(np.float32)
    keys[:, [3, 70]] += np.array([60.0, -85.0], np.float32)   # persistent outlier channels
    keys = keys.astype(np.float16)
    q = (rng.standard_normal(128) / math.sqrt(128)).astype(np.float64)
    per_channel, per_token = both(keys)
    kf = keys.astype(np.float64)
    assert np.abs(per_channel - kf).mean() < np.abs(per_token - kf).mean()
    assert np.abs((per_channel - kf) @ q).mean() < np.abs((per_token - kf) @ q).mean()


# ------------------------------------------------------------- axis ablation

def test_axis_ablation_errors_hand_case():
    """The four error measures of the axis ablation on a 4-token, 4-channel
    case worked out by hand (G = 4, B = 2).

    Keys K (rows are tokens): (1 2 -1 0), (1 2 -1 1), (1 2 -1 2), (1 2 -1 6);
    values 3 * I; q = (1, 0, 0, 1); alpha = ln 2, so exp(alpha s) = 2^s.
    * Per channel, columns 0-2 are constant (exact) and column 3 is the group
      (0, 1, 2, 6): step 2, token 1's quotient 0.5 rounds to the even code
      0, so K_hat - K is -1 at (1, 3) and 0 elsewhere.
    * Per token, rows 0-2 span -1..2 with step 1 (exact); row 3 spans -1..6:
      step fp16(7/3) = 1195/512, codes (1, 1, 0, 3), dequantized
      (683/512, 683/512, -1, 3073/512), error (171, -341, 0, 1) / 512.
    * The values 3 * I are exact on either axis (groups {0, 3}, step 1).
    sum |K| = 25, ||K||_F^2 = 65, K q = (1, 2, 3, 7).  The unquantized
    attention weights are (2, 4, 8, 128) / 142 and the output is 3 times
    them, so the output error is the relative error of the weights: per
    channel the scores become (1, 1, 3, 7), weights (2, 2, 8, 128) / 140;
    per token (1, 2, 3, 7 + 43/128)."""
    from oracle import axis_ablation as ab

    k = np.array([[1, 2, -1, 0], [1, 2, -1, 1], [1, 2, -1, 2], [1, 2, -1, 6]], np.float16)
    v = (3 * np.eye(4)).astype(np.float16)
    q = np.array([1, 0, 0, 1], np.float16)

    def norm(x):
        return math.sqrt(sum(float(a) ** 2 for a in x))

    p = [Fraction(x, 142) for x in (2, 4, 8, 128)]
    p_ch = [Fraction(x, 140) for x in (2, 2, 8, 128)]
    t = 128 * 2 ** (43 / 128)
    p_tok = [x / (14 + t) for x in (2, 4, 8, t)]
    want = {
        "channel": {"key_mean": 1 / 25, "key": 1 / math.sqrt(65), "score": 1 / math.sqrt(63),
                    "output": norm([a - b for a, b in zip(p_ch, p)]) / norm(p)},
        "token": {"key_mean": 513 / 12800, "key": math.sqrt(171 ** 2 + 341 ** 2 + 1) / 512 / math.sqrt(65),
                  "score": (172 / 512) / math.sqrt(63),
                  "output": norm([a - float(b) for a, b in zip(p_tok, p)]) / norm(p)},
    }
    for ka in ("channel", "token"):
        for va in ("channel", "token"):
            got = ab.errors(k, v, q, math.log(2), 4, 2, ka, va)
            for m, x in want[ka].items():
                assert got[m] == pytest.approx(x, rel=1e-12), (ka, va, m)
