"""Seeded synthetic workloads and the byte model.

This module holds no arithmetic of the method (no quantization, no
attention): it draws fp16 inputs and counts bytes.  Both the test suite (which
feeds the same arrays to the CPU oracle and to the GPU library) and the bench
use it.

Workloads are shaped like the pages' Llama-2-7B / 13B decode settings
(discosf KIVI tutorial, section 1 and section 4.2; unite.ai axis-selection
guide, systems section and the Llama-2-13B ablation): head_dim 128, fp16 K/V.
Keys carry a few persistent outlier channels per head, the structure the
guide's keys section describes (the same channels are large on every token);
values are plain N(0, 1) (values section: no channel outlier pattern).

Recipe (all draws from numpy ``Generator(PCG64(1000 + n))`` for workload n,
in this order: lengths, keys, values, query; drawn in fp32 and rounded to
fp16 with round-to-nearest-even):

* keys: N(0, 1).  Workload 1: 4 channels, chosen once without replacement,
  are multiplied by 50 on every token.  Workloads 2-5: per (sequence, head),
  n ~ U{1, 2, 3} channels chosen without replacement, each multiplied on
  every token by a factor of magnitude U[20, 100] and random sign.
* values: N(0, 1).
* query: N(0, 1) for workload 1 (sm_scale = 1/sqrt(128)); N(0, 1)/sqrt(128)
  for workloads 2-5 (sm_scale = 1).
* workload 4 lengths: context c ~ U{1024..8192}, window fill r ~ U{0..127},
  quantized tokens 32 * floor((c - r) / 32).
"""

from dataclasses import dataclass, field
import math

import numpy as np


@dataclass(frozen=True)
class Config:
    number: int
    name: str
    batch: int
    heads: int
    head_dim: int
    bits: int
    group: int
    residual: int
    context: int            # per-sequence tokens (upper bound for workload 4)
    window: int             # fp16 window tokens at decode time (workloads 1-3, 5)
    capacity: int           # quantized slots allocated per sequence
    sm_scale: float
    query_std: float
    description: str = field(default="", compare=False)


CONFIGS = {
    1: Config(1, "tiny_single_head", 1, 1, 128, 2, 32, 32, 256, 32, 256,
              1.0 / math.sqrt(128.0), 1.0,
              "batch 1, 1 head, 224 quantized + 32 fp16 window tokens, B=2 G=32 R=32"),
    2: Config(2, "llama2_7b_layer", 8, 32, 128, 2, 32, 128, 4096, 128, 4096,
              1.0, 1.0 / math.sqrt(128.0),
              "batch 8, 32 heads, 3968 quantized + 128 fp16 window tokens, B=2 G=32 R=128"),
    3: Config(3, "llama2_13b_layer", 16, 40, 128, 2, 32, 128, 2048, 128, 2048,
              1.0, 1.0 / math.sqrt(128.0),
              "batch 16, 40 heads, 1920 quantized + 128 fp16 window tokens, B=2 G=32 R=128"),
    4: Config(4, "ragged_serving", 64, 32, 128, 2, 32, 128, 8192, -1, 8192 + 128,
              1.0, 1.0 / math.sqrt(128.0),
              "batch 64, 32 heads, contexts U[1024,8192], window fill U[0,127], B=2 G=32 R=128"),
    5: Config(5, "long_context", 1, 32, 128, 2, 128, 128, 131072, 128, 131072,
              1.0, 1.0 / math.sqrt(128.0),
              "batch 1, 32 heads, 130944 quantized + 128 fp16 window tokens, G=128 R=128, B=2 or 4"),
}


@dataclass
class Workload:
    config: Config
    bits: int
    k: np.ndarray        # fp16 [batch, heads, max_tokens, D], zero beyond each length
    v: np.ndarray        # fp16 [batch, heads, max_tokens, D]
    q: np.ndarray        # fp16 [batch, heads, D]
    q_len: np.ndarray    # int32 [batch] quantized tokens at decode time
    r_len: np.ndarray    # int32 [batch] fp16 window tokens at decode time
    seed: int

    @property
    def lengths(self):
        return (self.q_len + self.r_len).astype(np.int32)

    def dims(self):
        c = self.config
        return dict(batch=int(self.q_len.shape[0]), heads=c.heads, head_dim=c.head_dim, bits=self.bits,
                    group=c.group, residual=c.residual, capacity=c.capacity)


def _lengths(cfg, rng):
    if cfg.number == 4:
        ctx = rng.integers(1024, 8192, size=cfg.batch, endpoint=True)
        fill = rng.integers(0, 127, size=cfg.batch, endpoint=True)
        ql = cfg.group * ((ctx - fill) // cfg.group)
        return ql.astype(np.int32), fill.astype(np.int32)
    ql = np.full(cfg.batch, cfg.context - cfg.window, np.int32)
    rl = np.full(cfg.batch, cfg.window, np.int32)
    return ql, rl


def generate(number, bits=None, batch=None):
    """Draw workload ``number`` (1-5).  ``bits`` overrides B (workload 5 runs
    at B=2 and B=4 on the same draws).  ``batch`` keeps only the first
    ``batch`` sequences of the same draws (lengths are drawn for the full
    batch first, so a prefix is identical to the full workload's prefix)."""
    cfg = CONFIGS[number]
    seed = 1000 + number
    rng = np.random.Generator(np.random.PCG64(seed))
    D, H = cfg.head_dim, cfg.heads
    ql, rl = _lengths(cfg, rng)
    nb = cfg.batch if batch is None else min(batch, cfg.batch)
    ql, rl = ql[:nb], rl[:nb]
    n = ql + rl
    T = int(n.max())
    k = np.zeros((nb, H, T, D), np.float16)
    v = np.zeros((nb, H, T, D), np.float16)
    if number == 1:
        fixed = rng.choice(D, size=4, replace=False)
    for b in range(nb):
        nk = rng.standard_normal((H, int(n[b]), D), dtype=np.float32)
        if number == 1:
            nk[:, :, fixed] *= np.float32(50.0)
        else:
            for h in range(H):
                cnt = int(rng.integers(1, 3, endpoint=True))
                ch = rng.choice(D, size=cnt, replace=False)
                mag = rng.uniform(20.0, 100.0, size=cnt).astype(np.float32)
                sign = rng.choice(np.array([-1.0, 1.0], np.float32), size=cnt)
                nk[h][:, ch] *= mag * sign
        k[b, :, :n[b]] = nk.astype(np.float16)
    for b in range(nb):
        v[b, :, :n[b]] = rng.standard_normal((H, int(n[b]), D), dtype=np.float32).astype(np.float16)
    q = (rng.standard_normal((nb, H, D), dtype=np.float32)
         * np.float32(cfg.query_std)).astype(np.float16)
    return Workload(config=cfg, bits=cfg.bits if bits is None else bits, k=k, v=v, q=q,
                    q_len=ql.astype(np.int32), r_len=rl.astype(np.int32), seed=seed)


def sink_tokens(w, n_sink, score=24.0):
    """fp16 attention-sink rows (k_sink, v_sink [batch, heads, n_sink, D])
    for workload ``w``, drawn from seed 3000 + workload number: keys
    N(0, 3^2) and values N(0, 1), except that sink token 0's key is
    ``score / sm_scale * q / |q|^2`` for its head, so that its score is about
    ``score`` (the large attention weight a sink token draws)."""
    cfg = w.config
    nb, H, D = w.q.shape
    rng = np.random.Generator(np.random.PCG64(3000 + cfg.number))
    ks = rng.standard_normal((nb, H, n_sink, D), dtype=np.float32) * np.float32(3.0)
    vs = rng.standard_normal((nb, H, n_sink, D), dtype=np.float32)
    if n_sink:
        q = w.q.astype(np.float64)
        n2 = np.maximum((q * q).sum(-1, keepdims=True), 1e-30)
        ks[:, :, 0] = (score / cfg.sm_scale * q / n2).astype(np.float32)
    return ks.astype(np.float16), vs.astype(np.float16)


# ---------------------------------------------------------------- byte model

def fp16_kv_cache_bytes(batch, seq_len, layers, hidden):
    """KV-cache size of an fp16 model (discosf KIVI tutorial, section 2.1):
    batch x sequence x 2 (K and V) x layers x hidden x 2 bytes."""
    return batch * seq_len * 2 * layers * hidden * 2


def decode_bytes_per_head(q_len, r_len, head_dim, bits, group):
    """Algorithmic HBM bytes one decode call must move for one
    (sequence, head): K and V codes, K zero+scale per group, V zero+scale
    per token group, the fp16 window K and V, the fp16 query, the fp32 output."""
    D = head_dim
    codes = 2 * q_len * D * bits // 8
    k_meta = (q_len // group) * D * 4
    v_meta = q_len * (D // group) * 4
    window = 2 * r_len * D * 2
    return codes + k_meta + v_meta + window + D * 2 + D * 4


def decode_bytes(q_len, r_len, heads, head_dim, bits, group):
    """Sum of ``decode_bytes_per_head`` over a batch (per-sequence lengths)."""
    return sum(heads * decode_bytes_per_head(int(a), int(b), head_dim, bits, group)
               for a, b in zip(np.asarray(q_len), np.asarray(r_len)))


def flush_bytes_per_head(residual, head_dim, bits, group):
    """Algorithmic bytes of flushing one full window of one (sequence, head):
    read R fp16 K and V tokens, write their codes and zero/scale arrays."""
    D = head_dim
    read = 2 * residual * D * 2
    write = 2 * residual * D * bits // 8 + (residual // group) * D * 4 + residual * (D // group) * 4
    return read + write


def flush_write_bytes_per_head(residual, head_dim, bits, group):
    """The write part of ``flush_bytes_per_head``: codes and zero/scale arrays."""
    D = head_dim
    return 2 * residual * D * bits // 8 + (residual // group) * D * 4 + residual * (D // group) * 4


def step_bytes(q_len, r_start, heads, head_dim, bits, group, residual):
    """Algorithmic bytes of one whole step done in one kernel, over a batch:
    the decode's bytes over the window with the appended token in it (that
    token is read from the new-token input instead of the window), writing
    the new K and V rows into the window, and, for every sequence whose
    window the append fills, the flush's writes (the window it quantizes is
    the one the decode reads)."""
    total = decode_bytes(q_len, np.asarray(r_start) + 1, heads, head_dim, bits, group)
    for r in np.asarray(r_start):
        total += heads * 2 * head_dim * 2
        if int(r) + 1 == residual:
            total += heads * flush_write_bytes_per_head(residual, head_dim, bits, group)
    return int(total)


def append_bytes_per_head(head_dim):
    """Algorithmic bytes of appending one token to one (sequence, head):
    read and write one fp16 K row and one fp16 V row."""
    return 2 * 2 * head_dim * 2
