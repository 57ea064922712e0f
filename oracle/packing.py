"""Packing of B-bit codes into the library's uint32 tile layout (oracle).

Test infrastructure only (see ``oracle/__init__.py``).

The pages fix no layout; this follows the layout documented in the library's
public header: codes live in tiles of G consecutive tokens; inside a tile the
words are ordered [word w][token t]; word (w, t) holds the codes of channels
w*(32/B) + i, i = 0 .. 32/B - 1, of token t, channel w*(32/B)+i at bits
[i*B, i*B + B), least significant first.
"""

import numpy as np


def pack_tiles(codes, group, bits):
    """codes: uint8 [L, D] (L a multiple of group) -> uint32 [L/G, W, G]."""
    L, D = codes.shape
    per_word = 32 // bits
    if L % group or D % per_word:
        raise ValueError("bad shape for packing")
    if codes.size and int(codes.max()) >= (1 << bits):
        raise ValueError("code out of range")
    n_words = D // per_word
    c = codes.astype(np.uint32).reshape(L // group, group, n_words, per_word)
    words = np.zeros((L // group, group, n_words), dtype=np.uint32)
    for i in range(per_word):
        words |= c[..., i] << np.uint32(i * bits)
    return np.ascontiguousarray(words.transpose(0, 2, 1))


def unpack_tiles(words, bits):
    """uint32 [T, W, G] -> codes uint8 [T*G, W*(32/B)] (inverse of pack)."""
    n_tiles, n_words, group = words.shape
    per_word = 32 // bits
    mask = np.uint32((1 << bits) - 1)
    w = words.transpose(0, 2, 1)                      # [tile, t, w]
    out = np.empty((n_tiles, group, n_words, per_word), dtype=np.uint8)
    for i in range(per_word):
        out[..., i] = (w >> np.uint32(i * bits)) & mask
    return out.reshape(n_tiles * group, n_words * per_word)
