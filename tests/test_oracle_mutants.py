"""Plant plausible mistakes in the oracle (CPU only) and check that the pins
in ``test_oracle.py`` catch every one of them.

Each mutant replaces one oracle function with a subtly wrong version (a wrong
rounding, a dropped term, a transposed axis, a wrong bit order ...).  The
test then runs the pins that should notice and requires at least one of them
to fail.  This shows the pins are strong enough that a slip anywhere in the
oracle would not go unnoticed.
"""

import numpy as np
import pytest

import oracle.attention as oatt
import oracle.axis_ablation as oab
import oracle.cache as ocache
import oracle.packing as opack
import oracle.quantizer as oq
import tests.test_oracle as pins

F32 = np.float32


def _quant(rounding=np.rint, levels_of=lambda b: 2 ** b - 1, zero_from_max=False,
           keep_neg_zero=False, reciprocal=False):
    def quantize_groups(x, bits):
        xf = np.asarray(x).astype(F32)
        levels = F32(levels_of(bits))
        mn = xf.min(-1) if keep_neg_zero else xf.min(-1) + F32(0)
        mx = xf.max(-1)
        step = ((mx - mn) / levels).astype(np.float16)
        s = step.astype(F32)
        ss = np.where(s != 0, s, F32(1))
        if reciprocal:
            qt = (xf - mn[..., None]) * (F32(1) / ss[..., None])
        else:
            qt = (xf - mn[..., None]) / ss[..., None]
        c = np.clip(rounding(qt), 0, F32(2 ** bits - 1))
        c = np.where(s[..., None] != 0, c, 0).astype(np.uint8)
        z = (mx if zero_from_max else mn).astype(np.float16)
        return c, z, step
    return quantize_groups


def _keys_per_token(k, group, bits):
    L, D = k.shape
    rows = k.reshape(L, D // group, group)
    c, z, s = oq.quantize_groups(rows, bits)
    return c.reshape(L, D), z[: L // group].reshape(L // group, -1).repeat(group, 1)[:, :D], \
        s[: L // group].reshape(L // group, -1).repeat(group, 1)[:, :D]


def _pack_msb_first(codes, group, bits):
    L, D = codes.shape
    per_word = 32 // bits
    c = codes.astype(np.uint32).reshape(L // group, group, D // per_word, per_word)
    words = np.zeros((L // group, group, D // per_word), np.uint32)
    for i in range(per_word):
        words |= c[..., i] << np.uint32(32 - bits - i * bits)
    return np.ascontiguousarray(words.transpose(0, 2, 1))


def _pack_token_major(codes, group, bits):
    L, D = codes.shape
    per_word = 32 // bits
    c = codes.astype(np.uint32).reshape(L // group, group, D // per_word, per_word)
    words = np.zeros((L // group, group, D // per_word), np.uint32)
    for i in range(per_word):
        words |= c[..., i] << np.uint32(i * bits)
    return np.ascontiguousarray(words).reshape(L // group, D // per_word, group)


def _attention_no_alpha(q, k, v, alpha):
    return _ATT(q, k, v, 1.0)


def _attention_keys_as_values(q, k, v, alpha):
    return _ATT(q, k, k, alpha)


def _attention_no_normalise(q, k, v, alpha):
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    if k.shape[0] == 0:
        return np.zeros(q.shape[0])
    s = alpha * (k @ q)
    return np.exp(s - s.max()) @ v


def _dequant_values_no_zero(codes, zero, scale, group):
    return codes.astype(np.float64) * np.repeat(scale.astype(np.float64), group, axis=1)


def _dequant_keys_wrong_group_axis(codes, zero, scale, group):
    z = np.tile(zero.astype(np.float64), (group, 1))
    s = np.tile(scale.astype(np.float64), (group, 1))
    return z + codes.astype(np.float64) * s


def _merge_without_rescale(parts):
    parts = [p for p in parts if p[1] > 0]
    return sum(a for _, _, a in parts) / sum(l for _, l, _ in parts)


def _tile_token_major(a, group):
    n, ng = a.shape
    return np.ascontiguousarray(a.reshape(n // group, group, ng))


def _untile_token_major(a):
    t, group, ng = a.shape
    return a.reshape(t * group, ng)


def _untile_group_major_misread(a):
    # reads the tiles as if they were token-major
    t, ng, group = a.shape
    return a.reshape(t * group, ng)


_ERRORS = oab.errors


def _errors_score_undivided(k, v, q, alpha, group, bits, k_axis, v_axis):
    e = _ERRORS(k, v, q, alpha, group, bits, k_axis, v_axis)
    kf, qf = k.astype(np.float64), np.asarray(q, np.float64)
    e["score"] *= float(np.linalg.norm(kf @ qf))
    return e


def _errors_output_over_quantized(k, v, q, alpha, group, bits, k_axis, v_axis):
    e = _ERRORS(k, v, q, alpha, group, bits, k_axis, v_axis)
    kf, vf, qf = k.astype(np.float64), v.astype(np.float64), np.asarray(q, np.float64)
    kh = oab.quantize_axis(k, k_axis, group, bits)
    vh = oab.quantize_axis(v, v_axis, group, bits)
    ref, got = oatt.attention(qf, kf, vf, alpha), oatt.attention(qf, kh, vh, alpha)
    e["output"] = float(np.linalg.norm(got - ref) / np.linalg.norm(got))
    return e


_ATT = oatt.attention
_ORIG_FLUSH = ocache.Cache.flush


def _flush_keeps_window(self):
    r = self.r_len.copy()
    _ORIG_FLUSH(self)
    self.r_len[:] = np.where(r == self.R, self.R, self.r_len)


QUANT_PINS = ["test_quantizer_hand_cases", "test_quantizer_matches_exact_brute_force",
              "test_error_at_most_half_step", "test_min_maps_to_zero_and_max_to_top_code",
              "test_constant_groups_reconstruct_exactly", "test_step_formula_is_range_over_levels"]
AXIS_PINS = ["test_key_and_value_axes_are_transposes", "test_key_groups_are_per_channel_over_tokens"]
PACK_PINS = ["test_packing_hand_cases"]
ATT_PINS = ["test_attention_closed_form", "test_attention_matches_textbook_loops",
            "test_residual_only_cache_is_exact_fp16_attention",
            "test_zero_query_gives_mean_of_dequantized_values"]
STREAM_PINS = ["test_streaming_equals_bulk"]

MUTANTS = [
    ("floor instead of round-to-nearest", oq, "quantize_groups", _quant(rounding=np.floor), QUANT_PINS),
    ("round half away from zero", oq, "quantize_groups",
     _quant(rounding=lambda a: np.floor(a + F32(0.5))), QUANT_PINS),
    ("2^B levels instead of 2^B - 1", oq, "quantize_groups", _quant(levels_of=lambda b: 2 ** b), QUANT_PINS),
    ("zero-point taken from the maximum", oq, "quantize_groups", _quant(zero_from_max=True), QUANT_PINS),
    ("-0 zero-point kept", oq, "quantize_groups", _quant(keep_neg_zero=True), QUANT_PINS),
    ("keys grouped per token", oq, "quantize_keys", _keys_per_token, AXIS_PINS),
    ("codes packed most significant first", opack, "pack_tiles", _pack_msb_first, PACK_PINS),
    ("tile stored token-major", opack, "pack_tiles", _pack_token_major, PACK_PINS),
    ("sm_scale dropped", oatt, "attention", _attention_no_alpha, ATT_PINS),
    ("keys used as values", oatt, "attention", _attention_keys_as_values, ATT_PINS),
    ("softmax not normalised", oatt, "attention", _attention_no_normalise, ATT_PINS),
    ("value zero-point dropped", oq, "dequantize_values", _dequant_values_no_zero,
     ["test_dequantization_is_exact", "test_constant_groups_reconstruct_exactly"]),
    ("key groups repeated along the wrong axis", oq, "dequantize_keys", _dequant_keys_wrong_group_axis,
     ["test_dequantization_is_exact", "test_attention_matches_textbook_loops"]),
    ("merge without exp(m_j - M) rescaling", oatt, "merge", _merge_without_rescale,
     ["test_split_merge_equals_single_pass"]),
    ("flush keeps the window length", ocache.Cache, "flush", _flush_keeps_window, STREAM_PINS),
    ("value tiles stored and read token-major", ocache, ("tile_value_groups", "untile_value_groups"),
     (_tile_token_major, _untile_token_major), ["test_value_group_tile_order_hand_cases"]),
    ("value tiles read token-major", ocache, "untile_value_groups", _untile_group_major_misread,
     ["test_value_group_tile_order_hand_cases"]),
    ("ablation score error without its denominator", oab, "errors", _errors_score_undivided,
     ["test_axis_ablation_errors_hand_case"]),
    ("ablation output error relative to the quantized output", oab, "errors",
     _errors_output_over_quantized, ["test_axis_ablation_errors_hand_case"]),
]


def _run(name, golden_dir):
    fn = getattr(pins, name)
    params = {"golden_dir": golden_dir}
    mark = getattr(fn, "pytestmark", [])
    cases = [{}]
    for m in mark:
        if m.name == "parametrize":
            argnames = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) else m.args[0]
            cases = [dict(zip(argnames, v if isinstance(v, tuple) else (v,))) for v in m.args[1]]
    for case in cases:
        kw = dict(case)
        if "golden_dir" in fn.__code__.co_varnames[:fn.__code__.co_argcount]:
            kw.update(params)
        fn(**kw)


@pytest.mark.parametrize("label,module,attr,mutant,pin_names", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(label, module, attr, mutant, pin_names, monkeypatch, golden_dir):
    if isinstance(attr, tuple):  # a mistake made the same way in several functions
        for a, m in zip(attr, mutant):
            monkeypatch.setattr(module, a, m)
    else:
        monkeypatch.setattr(module, attr, mutant)
    caught = []
    for name in pin_names:
        try:
            with np.errstate(all="ignore"):
                _run(name, golden_dir)
        except (AssertionError, ValueError, IndexError, TypeError):
            caught.append(name)
    assert caught, f"no pin caught the planted mistake: {label}"
