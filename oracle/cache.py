"""Streaming quantized KV cache, in the library's buffer layouts (oracle).

Test infrastructure only (see ``oracle/__init__.py``).

Streaming rule (discosf KIVI tutorial, section 3.1; unite.ai axis-selection
guide, systems section): the newest tokens are kept in an fp16 window; once
R tokens have accumulated, they are quantized group-wise (keys as R/G groups
of G tokens per channel, values per token) and the window is emptied.  Key
groups therefore always start at token positions that are multiples of G.
A prompt of l tokens is split as in the tutorial's section 3.1 sketch:
r = l mod G tokens stay in fp16 and the first l - r are quantized, unless an
explicit window size is given.

Buffer layouts and length rules are the ones the library's public header
documents (tiles of G tokens, fp16 zero/scale arrays, int32 lengths, sticky
status bits), so the oracle's buffers can be compared with the GPU's byte for
byte.  Everything is per (sequence, head) and plain numpy.
"""

import numpy as np

from .attention import attention
from .packing import pack_tiles, unpack_tiles
from .quantizer import (dequantize_keys, dequantize_values, quantize_keys,
                        quantize_values)

ST_RESIDUAL_FULL = 0x1
ST_CAPACITY = 0x2
ST_BAD_LENGTH = 0x4


def encode_tokens(k, v, group, bits):
    """Quantize n fp16 tokens (n a multiple of G) of one (sequence, head).

    k, v: fp16 [n, D].  Returns a dict with k_codes/v_codes uint32
    [n/G, W, G], k_zero/k_scale fp16 [n/G, D] and v_zero/v_scale fp16
    [n/G, D/G, G] (value groups stored per tile of G tokens, group-major).
    """
    ck, zk, sk = quantize_keys(k, group, bits)
    cv, zv, sv = quantize_values(v, group, bits)
    return dict(k_codes=pack_tiles(ck, group, bits), k_zero=zk, k_scale=sk,
                v_codes=pack_tiles(cv, group, bits), v_zero=tile_value_groups(zv, group),
                v_scale=tile_value_groups(sv, group))


def tile_value_groups(a, group):
    """Per-token value-group array [n, D/G] -> tiles [n/G, D/G, G]."""
    n, ng = a.shape
    return np.ascontiguousarray(a.reshape(n // group, group, ng).transpose(0, 2, 1))


def untile_value_groups(a):
    """Tiles [T, D/G, G] -> per-token value-group array [T*G, D/G]."""
    t, ng, group = a.shape
    return a.transpose(0, 2, 1).reshape(t * group, ng)


def context(state, group, bits):
    """Dequantized context of one (sequence, head): fp64 K [T, D], V [T, D]
    with the q_len quantized tokens first, then the r_len window tokens."""
    ql, rl = int(state["q_len"]), int(state["r_len"])
    nt = ql // group
    ck = unpack_tiles(state["k_codes"][:nt], bits)
    cv = unpack_tiles(state["v_codes"][:nt], bits)
    kq = dequantize_keys(ck, state["k_zero"][:nt], state["k_scale"][:nt], group)
    vq = dequantize_values(cv, untile_value_groups(state["v_zero"][:nt]),
                           untile_value_groups(state["v_scale"][:nt]), group)
    kr = state["k_res"][:rl].astype(np.float64)
    vr = state["v_res"][:rl].astype(np.float64)
    return np.concatenate([kq, kr], axis=0), np.concatenate([vq, vr], axis=0)


def head_state(k, v, q_len, r_len, group, bits, capacity, residual):
    """Cache state of one (sequence, head) holding tokens k[:q_len+r_len]:
    the first q_len quantized, the next r_len in the window (bulk form)."""
    D = k.shape[1]
    W = D * bits // 32
    st = dict(
        k_codes=np.zeros((capacity // group, W, group), np.uint32),
        v_codes=np.zeros((capacity // group, W, group), np.uint32),
        k_zero=np.zeros((capacity // group, D), np.float16),
        k_scale=np.zeros((capacity // group, D), np.float16),
        v_zero=np.zeros((capacity // group, D // group, group), np.float16),
        v_scale=np.zeros((capacity // group, D // group, group), np.float16),
        k_res=np.zeros((residual, D), np.float16),
        v_res=np.zeros((residual, D), np.float16),
        q_len=q_len, r_len=r_len)
    if q_len:
        enc = encode_tokens(k[:q_len], v[:q_len], group, bits)
        nt = q_len // group
        for name in ("k_codes", "v_codes", "k_zero", "k_scale", "v_zero", "v_scale"):
            st[name][:nt] = enc[name]
    st["k_res"][:r_len] = k[q_len:q_len + r_len]
    st["v_res"][:r_len] = v[q_len:q_len + r_len]
    return st


class Cache:
    """Whole-batch cache with the library's entry points as methods."""

    def __init__(self, batch, heads, head_dim, bits, group, residual, capacity):
        self.batch, self.heads, self.D = batch, heads, head_dim
        self.bits, self.G, self.R, self.cap = bits, group, residual, capacity
        W = head_dim * bits // 32
        nt = capacity // group
        self.k_codes = np.zeros((batch, heads, nt, W, group), np.uint32)
        self.v_codes = np.zeros((batch, heads, nt, W, group), np.uint32)
        self.k_zero = np.zeros((batch, heads, nt, head_dim), np.float16)
        self.k_scale = np.zeros((batch, heads, nt, head_dim), np.float16)
        self.v_zero = np.zeros((batch, heads, nt, head_dim // group, group), np.float16)
        self.v_scale = np.zeros((batch, heads, nt, head_dim // group, group), np.float16)
        self.k_res = np.zeros((batch, heads, residual, head_dim), np.float16)
        self.v_res = np.zeros((batch, heads, residual, head_dim), np.float16)
        self.q_len = np.zeros(batch, np.int32)
        self.r_len = np.zeros(batch, np.int32)
        self.status = 0

    def _store(self, b, h, pos, k, v):
        enc = encode_tokens(k, v, self.G, self.bits)
        t0, nt = pos // self.G, k.shape[0] // self.G
        for name in ("k_codes", "k_zero", "k_scale", "v_codes", "v_zero", "v_scale"):
            getattr(self, name)[b, h, t0:t0 + nt] = enc[name]

    def prefill(self, k, v, lens, res=None):
        """k, v: fp16 [batch, heads, src_len, D]; lens/res: int [batch]."""
        src_len = k.shape[2]
        for b in range(self.batch):
            n = int(lens[b])
            r = n % self.G if res is None else int(res[b])
            self.q_len[b] = self.r_len[b] = 0
            if n < 0 or n > src_len or r < 0 or r > self.R or r > n or (n - r) % self.G:
                self.status |= ST_BAD_LENGTH
                continue
            if n - r > self.cap:
                self.status |= ST_CAPACITY
                continue
            for h in range(self.heads):
                if n - r:
                    self._store(b, h, 0, k[b, h, :n - r], v[b, h, :n - r])
                self.k_res[b, h, :r] = k[b, h, n - r:n]
                self.v_res[b, h, :r] = v[b, h, n - r:n]
            self.q_len[b], self.r_len[b] = n - r, r

    def append(self, k_new, v_new):
        """k_new, v_new: fp16 [batch, heads, D]."""
        for b in range(self.batch):
            r = int(self.r_len[b])
            if r < 0:
                self.status |= ST_BAD_LENGTH
                continue
            if r >= self.R:
                self.status |= ST_RESIDUAL_FULL
                continue
            self.k_res[b, :, r] = k_new[b]
            self.v_res[b, :, r] = v_new[b]
            self.r_len[b] = r + 1

    def flush(self):
        for b in range(self.batch):
            if int(self.r_len[b]) != self.R:
                continue
            q = int(self.q_len[b])
            if q + self.R > self.cap:
                self.status |= ST_CAPACITY
                continue
            for h in range(self.heads):
                self._store(b, h, q, self.k_res[b, h], self.v_res[b, h])
            self.q_len[b] = q + self.R
            self.r_len[b] = 0

    def head(self, b, h):
        return dict(k_codes=self.k_codes[b, h], v_codes=self.v_codes[b, h],
                    k_zero=self.k_zero[b, h], k_scale=self.k_scale[b, h],
                    v_zero=self.v_zero[b, h], v_scale=self.v_scale[b, h],
                    k_res=self.k_res[b, h], v_res=self.v_res[b, h],
                    q_len=self.q_len[b], r_len=self.r_len[b])

    def lengths_valid(self, b):
        ql, rl = int(self.q_len[b]), int(self.r_len[b])
        return 0 <= ql <= self.cap and ql % self.G == 0 and 0 <= rl <= self.R

    def decode(self, q, alpha):
        """q: fp16 [batch, heads, D] -> fp64 [batch, heads, D]."""
        out = np.zeros((self.batch, self.heads, self.D), np.float64)
        for b in range(self.batch):
            if not self.lengths_valid(b):
                self.status |= ST_BAD_LENGTH
                continue
            for h in range(self.heads):
                kk, vv = context(self.head(b, h), self.G, self.bits)
                out[b, h] = attention(q[b, h], kk, vv, alpha)
        return out


def decode_head(q, state, alpha, group, bits):
    """Decode output (fp64 [D]) of one (sequence, head) cache state."""
    kk, vv = context(state, group, bits)
    return attention(q, kk, vv, alpha)


def value_queue(v, residual, group, bits):
    """Value-queue variant (discosf KIVI tutorial, section 3.2): value tokens
    enter an fp16 queue one at a time; whenever the queue holds more than R
    tokens, the oldest is popped and quantized on its own (per token, groups of
    G channels), so the newest R always stay fp16.  Returns the
    (codes, zero, scale) of each popped token in eviction order."""
    queue, evicted = [], []
    for t in range(v.shape[0]):
        queue.append(v[t])
        while len(queue) > residual:
            oldest = queue.pop(0)
            codes, zero, scale = quantize_values(oldest[None, :], group, bits)
            evicted.append((codes[0], zero[0], scale[0]))
    return evicted
