"""Axis ablation on the synthetic workloads (direction only, CPU).

The unite.ai axis-selection guide (keys section) groups keys per channel
because a few channels carry large magnitudes on every token; grouping them
per token lets those channels set the step of every group.  On the
Llama-2-7B-shaped workload (persistent outlier key channels) per-channel key
groups must give lower key error (mean absolute), lower score error and
lower attention-output error than per-token ones, at B=2 and B=4, whichever
axis the values use.  The guide's own figures need real activations; these
are the synthetic ones.

``python -m tests.test_axis_ablation`` prints the full table.
"""

import numpy as np
import pytest

from bit_kv_cache_decode_amd import workloads as wl
from oracle import axis_ablation as ab


def _heads(w, n, tokens, seed):
    rng = np.random.default_rng(seed)
    b = rng.integers(0, w.k.shape[0], n)
    h = rng.integers(0, w.k.shape[1], n)
    return [(w.k[i, j, :tokens], w.v[i, j, :tokens], w.q[i, j]) for i, j in zip(b, h)]


@pytest.mark.parametrize("bits", [2, 4])
def test_per_channel_keys_give_lower_score_and_output_error(bits):
    w = wl.generate(2, batch=2)
    res = ab.ablate(_heads(w, 4, 1024, 7), w.config.sm_scale, w.config.group, bits)
    for va in ab.AXES:
        ch, tok = res[("channel", va)], res[("token", va)]
        assert ch["key_mean"] < tok["key_mean"]
        assert ch["score"] < tok["score"]
        assert ch["output"] < tok["output"]


def test_axis_choice_of_values_leaves_key_errors_alone():
    w = wl.generate(2, batch=1)
    res = ab.ablate(_heads(w, 2, 512, 3), w.config.sm_scale, w.config.group, 2)
    for ka in ab.AXES:
        assert res[(ka, "channel")]["key"] == res[(ka, "token")]["key"]
        assert res[(ka, "channel")]["score"] == res[(ka, "token")]["score"]


def main():
    w = wl.generate(2)
    heads = _heads(w, 16, 3968, 99)
    for bits in (2, 4):
        print(f"Llama-2-7B-shaped layer, 16 sampled (sequence, head) pairs, 3968 tokens, "
              f"B={bits}, G={w.config.group}:")
        print(ab.table(ab.ablate(heads, w.config.sm_scale, w.config.group, bits)))
        print()


if __name__ == "__main__":
    main()
