"""Cache with a value queue (oracle): keys flushed R at a time, values
quantized one token at a time as they leave an fp16 queue of the newest R.

Test infrastructure only (see ``oracle/__init__.py``).

The discosf KIVI tutorial, section 3.2 (value cache management), keeps the
values in an fp16 queue: a new token's value enters the queue, and once the
queue holds more than R tokens its oldest value is taken out and quantized on
its own (per token, groups of G channels; unite.ai axis-selection guide,
values section).  Keys keep the rule of section 3.1: they collect in an fp16
window of up to R tokens that is quantized group-wise, R/G key groups of G
tokens per channel, when it is full.

Consequences for a sequence of T tokens (q_len quantized keys, r_len keys in
the window, T = q_len + r_len):

* the newest min(T, R) values are fp16; the first vq = max(0, T - R) are
  quantized, each token on its own, so the value codes, zero-points and steps
  of token t are exactly those the bulk per-token quantizer gives it;
* vq <= q_len always (r_len <= R), so the context splits into three runs:
  tokens [0, vq) with quantized keys and values, [vq, q_len) with quantized
  keys and fp16 values, [q_len, T) with fp16 keys and values.

Buffers are those of ``cache.Cache`` (the library's tile layouts), except
that ``v_res`` is a ring: the value of token t (t >= vq) is in slot t mod R.
Value tiles are filled a token at a time; positions past vq hold zeros.
"""

import numpy as np

from .attention import attention
from .cache import ST_BAD_LENGTH, ST_CAPACITY, ST_RESIDUAL_FULL, tile_value_groups, untile_value_groups
from .packing import pack_tiles, unpack_tiles
from .quantizer import dequantize_keys, dequantize_values, quantize_keys, quantize_values


def quantized_values(t_total, residual):
    """Values of a sequence of ``t_total`` tokens that have left the queue."""
    return max(0, int(t_total) - int(residual))


class ValueQueueCache:
    """Whole-batch cache with a value queue, the library's layouts."""

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
        self.v_res = np.zeros((batch, heads, residual, head_dim), np.float16)   # ring
        self.q_len = np.zeros(batch, np.int32)
        self.r_len = np.zeros(batch, np.int32)
        self.status = 0

    # -- storing
    def _store_keys(self, b, h, pos, k):
        codes, zero, scale = quantize_keys(k, self.G, self.bits)
        t0, nt = pos // self.G, k.shape[0] // self.G
        self.k_codes[b, h, t0:t0 + nt] = pack_tiles(codes, self.G, self.bits)
        self.k_zero[b, h, t0:t0 + nt] = zero
        self.k_scale[b, h, t0:t0 + nt] = scale

    def _store_value(self, b, h, t, v_row):
        """Quantize the value of token t (one token, D/G groups) into its
        place in the value tiles."""
        codes, zero, scale = quantize_values(v_row[None, :], self.G, self.bits)
        tile, pos = t // self.G, t % self.G
        block = np.zeros((self.G, self.D), np.uint8)
        block[pos] = codes[0]
        self.v_codes[b, h, tile, :, pos] = pack_tiles(block, self.G, self.bits)[0, :, pos]
        z = np.zeros((self.G, self.D // self.G), np.float16)
        s = np.zeros((self.G, self.D // self.G), np.float16)
        z[pos], s[pos] = zero[0], scale[0]
        self.v_zero[b, h, tile, :, pos] = tile_value_groups(z, self.G)[0, :, pos]
        self.v_scale[b, h, tile, :, pos] = tile_value_groups(s, self.G)[0, :, pos]

    def _store_values(self, b, h, vals):
        """Quantize the values of tokens [0, n) (per token, as _store_value
        does one at a time) into the value tiles; positions past n in the
        last tile stay zero."""
        n = vals.shape[0]
        codes, zero, scale = quantize_values(vals, self.G, self.bits)
        nt = -(-n // self.G)
        pad = nt * self.G - n
        codes = np.concatenate([codes, np.zeros((pad, self.D), np.uint8)])
        zero = np.concatenate([zero, np.zeros((pad, self.D // self.G), np.float16)])
        scale = np.concatenate([scale, np.zeros((pad, self.D // self.G), np.float16)])
        self.v_codes[b, h, :nt] = pack_tiles(codes, self.G, self.bits)
        self.v_zero[b, h, :nt] = tile_value_groups(zero, self.G)
        self.v_scale[b, h, :nt] = tile_value_groups(scale, self.G)

    def lengths_valid(self, b):
        ql, rl = int(self.q_len[b]), int(self.r_len[b])
        return 0 <= ql <= self.cap and ql % self.G == 0 and 0 <= rl <= self.R

    # -- the entry points
    def prefill(self, k, v, lens, res=None):
        """k, v: fp16 [batch, heads, src_len, D]; the key split of
        ``cache.Cache.prefill`` (r = len mod G unless given); values: the
        first max(0, len - R) quantized per token, the rest in the ring."""
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
            vq = quantized_values(n, self.R)
            for h in range(self.heads):
                if n - r:
                    self._store_keys(b, h, 0, k[b, h, :n - r])
                self.k_res[b, h, :r] = k[b, h, n - r:n]
                if vq:
                    self._store_values(b, h, v[b, h, :vq])
                for t in range(vq, n):
                    self.v_res[b, h, t % self.R] = v[b, h, t]
            self.q_len[b], self.r_len[b] = n - r, r

    def append(self, k_new, v_new):
        """k_new, v_new: fp16 [batch, heads, D].  The key goes to window slot
        r_len; the value enters the queue: once R values are queued, the
        oldest (token T - R, ring slot T mod R) is quantized and its slot
        takes the new value."""
        for b in range(self.batch):
            r = int(self.r_len[b])
            if r < 0 or not self.lengths_valid(b):
                self.status |= ST_BAD_LENGTH
                continue
            if r >= self.R:
                self.status |= ST_RESIDUAL_FULL
                continue
            T = int(self.q_len[b]) + r
            slot = T % self.R
            for h in range(self.heads):
                if T >= self.R:
                    self._store_value(b, h, T - self.R, self.v_res[b, h, slot])
                self.v_res[b, h, slot] = v_new[b, h]
                self.k_res[b, h, r] = k_new[b, h]
            self.r_len[b] = r + 1

    def flush(self):
        """Keys only: a full key window becomes R/G key groups."""
        for b in range(self.batch):
            if int(self.r_len[b]) != self.R:
                continue
            q = int(self.q_len[b])
            if q < 0 or q % self.G:
                self.status |= ST_BAD_LENGTH
                continue
            if q + self.R > self.cap:
                self.status |= ST_CAPACITY
                continue
            for h in range(self.heads):
                self._store_keys(b, h, q, self.k_res[b, h])
            self.q_len[b] = q + self.R
            self.r_len[b] = 0

    def head(self, b, h):
        return dict(k_codes=self.k_codes[b, h], v_codes=self.v_codes[b, h],
                    k_zero=self.k_zero[b, h], k_scale=self.k_scale[b, h],
                    v_zero=self.v_zero[b, h], v_scale=self.v_scale[b, h],
                    k_res=self.k_res[b, h], v_res=self.v_res[b, h],
                    q_len=self.q_len[b], r_len=self.r_len[b])

    def decode(self, q, alpha):
        """q: fp16 [batch, heads, D] -> fp64 [batch, heads, D]."""
        out = np.zeros((self.batch, self.heads, self.D), np.float64)
        for b in range(self.batch):
            if not self.lengths_valid(b):
                self.status |= ST_BAD_LENGTH
                continue
            for h in range(self.heads):
                kk, vv = context(self.head(b, h), self.G, self.bits, self.R)
                out[b, h] = attention(q[b, h], kk, vv, alpha)
        return out


def context(state, group, bits, residual):
    """Keys and values of one (sequence, head) of a value-queue cache in
    token order, fp64: keys dequantized for [0, q_len) then the key window;
    values dequantized for [0, vq) then fp16 from the ring for [vq, T)."""
    ql, rl = int(state["q_len"]), int(state["r_len"])
    T = ql + rl
    vq = quantized_values(T, residual)
    nk = ql // group
    kq = dequantize_keys(unpack_tiles(state["k_codes"][:nk], bits), state["k_zero"][:nk],
                         state["k_scale"][:nk], group)
    kk = np.concatenate([kq, state["k_res"][:rl].astype(np.float64)], axis=0)
    nv = -(-vq // group)
    cv = unpack_tiles(state["v_codes"][:nv], bits)[:vq]
    zv = untile_value_groups(state["v_zero"][:nv])[:vq]
    sv = untile_value_groups(state["v_scale"][:nv])[:vq]
    vqd = dequantize_values(cv, zv, sv, group)
    ring = np.array([state["v_res"][t % residual] for t in range(vq, T)], np.float64).reshape(-1, kk.shape[1])
    return kk, np.concatenate([vqd, ring], axis=0)


def decode_head(q, state, alpha, group, bits, residual):
    """Decode output (fp64 [D]) of one (sequence, head) value-queue state."""
    kk, vv = context(state, group, bits, residual)
    return attention(q, kk, vv, alpha)


def head_state(k, v, n, r, group, bits, capacity, residual):
    """Value-queue cache state of one (sequence, head) holding tokens
    k[:n], v[:n] with r keys in the window (the bulk form of prefill)."""
    c = ValueQueueCache(1, 1, k.shape[1], bits, group, residual, capacity)
    c.prefill(k[None, None], v[None, None], np.array([n]), np.array([r]))
    if c.status:
        raise ValueError("impossible lengths for a value-queue state")
    st = c.head(0, 0)
    return {n_: (np.array(x) if isinstance(x, np.ndarray) else int(x)) for n_, x in st.items()}
