"""Host-side checks of the C ABI (no GPU needed): the shared library loads,
exports every function include/kivi.h declares, validates dimensions, sizes
the workspace and rejects bad arguments before touching the device."""

import ctypes
import os
import re

import pytest

from bit_kv_cache_decode_amd import kivi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kivi.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kivi_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert len(names) >= 8
    L = kivi.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(kivi.EXPORTS) == names


def test_binding_declares_argument_types_of_every_entry_point():
    """ctypes passes an undeclared argument as a C int: a device pointer would
    arrive cut to 32 bits.  Every entry point's argument list is declared,
    with one ctypes type per parameter of its C declaration."""
    L = kivi.lib()
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for name in kivi.EXPORTS:
        types = getattr(L, name).argtypes
        assert types is not None, name
        params = re.search(name + r"\s*\(([^)]*)\)", text).group(1)
        n = 0 if params.strip() in ("", "void") else params.count(",") + 1
        assert len(types) == n, (name, len(types), n)
        # pointer parameters are declared as pointers, never as integers
        for t, prm in zip(types, params.split(",")):
            if "*" in prm:
                assert t is ctypes.c_void_p or t is ctypes.c_char_p or \
                    issubclass(t, ctypes._Pointer), (name, prm)


def test_validate_dims_codes():
    ok = kivi.make_dims(8, 32, 128, 2, 32, 128, 4096)
    assert kivi.validate_dims(ok) == kivi.KIVI_OK
    bad = [
        (0, 32, 128, 2, 32, 128, 4096),      # batch
        (8, 32, 128, 3, 32, 128, 4096),      # bits
        (8, 32, 100, 2, 32, 128, 4096),      # G does not divide head_dim
        (8, 32, 128, 2, 32, 100, 4096),      # G does not divide R
        (8, 32, 128, 2, 32, 128, 4016),      # G does not divide capacity
        (8, 32, 128, 2, 32, 128, -32),       # negative capacity
        (8, 32, 8, 2, 8, 8, 64),             # head_dim * bits not a multiple of 32
    ]
    for args in bad:
        assert kivi.validate_dims(kivi.make_dims(*args)) == kivi.KIVI_EINVAL, args
    # valid but not compiled: head_dim 64, group 16
    assert kivi.decode_splits(kivi.make_dims(8, 32, 64, 2, 32, 128, 4096)) == kivi.KIVI_EUNSUPPORTED
    assert kivi.decode_splits(kivi.make_dims(8, 32, 128, 4, 16, 128, 4096)) == kivi.KIVI_EUNSUPPORTED
    assert kivi.workspace_bytes(kivi.make_dims(8, 32, 64, 2, 32, 128, 4096)) == 0


@pytest.mark.parametrize("bits,bytes_per_token", [(2, 32), (4, 64), (8, 128)])
def test_capacity_limit_of_32_bit_buffer_offsets(bits, bytes_per_token):
    """One (sequence, head) region of the code arrays must stay below 2 GiB
    (the decode addresses it with 32-bit buffer offsets): the largest
    capacity below the limit is accepted, the first at it is refused as
    unsupported, not wrapped."""
    limit = (1 << 31) // bytes_per_token          # tokens whose codes fill 2 GiB
    below = limit - 128
    assert kivi.decode_splits(kivi.make_dims(1, 1, 128, bits, 128, 128, below)) >= 1
    assert kivi.decode_splits(kivi.make_dims(1, 1, 128, bits, 128, 128, limit)) == \
        kivi.KIVI_EUNSUPPORTED
    assert kivi.workspace_bytes(kivi.make_dims(1, 1, 128, bits, 128, 128, limit)) == 0


@pytest.mark.parametrize("dims,splits,step_kernels", [
    ((1, 1, 128, 2, 32, 32, 256), 1, 1),         # one workgroup does it all
    ((8, 32, 128, 2, 32, 128, 4096), 1, 1),      # one workgroup per (sequence, head) fills the chip
    ((16, 40, 128, 2, 32, 128, 2048), 1, 3),     # more pairs than compute units
    ((64, 32, 128, 2, 32, 128, 8320), 1, 3),     # many sequences: one workgroup each
    ((1, 32, 128, 2, 128, 128, 131072), 8, 3),   # long context: 8 workgroups per head
    ((1, 32, 128, 4, 128, 128, 131072), 8, 3),
    ((1, 1, 128, 2, 32, 32, 0), 1, 1),           # window only
    ((8, 32, 128, 8, 32, 128, 4096), 1, 3),      # 8 bits: one workgroup per head, step as three kernels
    ((1, 32, 128, 8, 128, 128, 131072), 8, 3),
    ((1, 1, 128, 2, 32, 4096, 1 << 24), 64, 3),  # capped at 64
])
def test_decode_plan(dims, splits, step_kernels):
    d = kivi.make_dims(*dims)
    assert kivi.decode_splits(d) == splits
    assert kivi.decode_step_kernels(d) == step_kernels
    bh = dims[0] * dims[1]
    ws = kivi.workspace_bytes(d)
    # partial states (4 + head_dim floats per split) plus one ticket per
    # (sequence, head), each on its own 256-byte line
    assert ws >= bh * splits * (4 + 128) * 4 + bh * 256
    assert ws % 256 == 0


def test_entry_points_reject_bad_arguments_without_a_device():
    L = kivi.lib()
    d = kivi.make_dims(2, 2, 128, 2, 32, 32, 256)
    fake = ctypes.c_void_p(0x1000)
    cs = kivi.CacheStruct(*([0x1000] * len(kivi.CacheStruct._fields_)))
    null_cache = kivi.CacheStruct()
    bad = kivi.make_dims(2, 2, 128, 3, 32, 32, 256)
    assert L.kivi_append_kv(ctypes.byref(bad), ctypes.byref(cs), fake, fake, None) == kivi.KIVI_EINVAL
    assert L.kivi_append_kv(ctypes.byref(d), ctypes.byref(null_cache), fake, fake, None) == kivi.KIVI_EINVAL
    assert L.kivi_append_kv(ctypes.byref(d), ctypes.byref(cs), None, fake, None) == kivi.KIVI_EINVAL
    assert L.kivi_flush_residual(ctypes.byref(bad), ctypes.byref(cs), None) == kivi.KIVI_EINVAL
    assert L.kivi_prefill(ctypes.byref(d), ctypes.byref(cs), fake, fake, 64, None, None, None) == kivi.KIVI_EINVAL
    assert L.kivi_prefill(ctypes.byref(d), ctypes.byref(cs), fake, fake, -1, fake, None, None) == kivi.KIVI_EINVAL
    need = kivi.workspace_bytes(d)
    assert L.kivi_decode_attn(ctypes.byref(d), ctypes.byref(cs), fake, fake, ctypes.c_float(1.0),
                              fake, ctypes.c_size_t(need - 1), None) == kivi.KIVI_ENOSPC
    assert L.kivi_decode_attn(ctypes.byref(d), ctypes.byref(cs), fake, fake, ctypes.c_float(float("nan")),
                              fake, ctypes.c_size_t(need), None) == kivi.KIVI_EINVAL
    assert L.kivi_decode_attn(ctypes.byref(d), ctypes.byref(cs), None, fake, ctypes.c_float(1.0),
                              fake, ctypes.c_size_t(need), None) == kivi.KIVI_EINVAL
    for base in (1.0, 0.5, float("nan"), float("inf")):
        assert L.kivi_decode_attn_rope(ctypes.byref(d), ctypes.byref(cs), fake, fake, ctypes.c_float(1.0),
                                       ctypes.c_double(base), fake, ctypes.c_size_t(need),
                                       None) == kivi.KIVI_EINVAL
    assert L.kivi_decode_attn_rope(ctypes.byref(d), ctypes.byref(cs), fake, fake, ctypes.c_float(1.0),
                                   ctypes.c_double(1e4), fake, ctypes.c_size_t(need - 1),
                                   None) == kivi.KIVI_ENOSPC
    # the sink decode: n_sink outside [0, 4096], a NULL sink with n_sink > 0,
    # a short workspace
    i32 = ctypes.c_int32
    c0 = ctypes.c_double(0.0)
    for n, ks, vs in ((-1, fake, fake), (4097, fake, fake), (4, None, fake), (4, fake, None)):
        assert L.kivi_decode_attn_sink(ctypes.byref(d), ctypes.byref(cs), ks, vs, i32(n), fake, fake,
                                       ctypes.c_float(1.0), c0, fake, ctypes.c_size_t(need),
                                       None) == kivi.KIVI_EINVAL
    assert L.kivi_decode_attn_sink(ctypes.byref(d), ctypes.byref(cs), fake, fake, i32(4), fake, fake,
                                   ctypes.c_float(float("nan")), c0, fake, ctypes.c_size_t(need),
                                   None) == kivi.KIVI_EINVAL
    # rope_base: 0 (none) or > 1 and finite
    for base in (1.0, 0.5, -3.0, float("nan"), float("inf")):
        assert L.kivi_decode_attn_sink(ctypes.byref(d), ctypes.byref(cs), fake, fake, i32(4), fake,
                                       fake, ctypes.c_float(1.0), ctypes.c_double(base), fake,
                                       ctypes.c_size_t(need), None) == kivi.KIVI_EINVAL
    for base in (0.0, 1e4):
        assert L.kivi_decode_attn_sink(ctypes.byref(d), ctypes.byref(cs), fake, fake, i32(4), fake,
                                       fake, ctypes.c_float(1.0), ctypes.c_double(base), fake,
                                       ctypes.c_size_t(need - 1), None) == kivi.KIVI_ENOSPC
    # the stream-read measurement aid: null, empty, unaligned or oddly sized
    # buffers and workgroup counts outside [1, 2^20]
    sz = ctypes.c_size_t
    assert L.kivi_stream_read(None, sz(1024), 4, fake, None) == kivi.KIVI_EINVAL
    assert L.kivi_stream_read(fake, sz(1024), 4, None, None) == kivi.KIVI_EINVAL
    assert L.kivi_stream_read(fake, sz(0), 4, fake, None) == kivi.KIVI_EINVAL
    assert L.kivi_stream_read(fake, sz(1000), 4, fake, None) == kivi.KIVI_EINVAL
    assert L.kivi_stream_read(ctypes.c_void_p(0x1008), sz(1024), 4, fake, None) == kivi.KIVI_EINVAL
    assert L.kivi_stream_read(fake, sz(1024), 0, fake, None) == kivi.KIVI_EINVAL
    assert L.kivi_stream_read(fake, sz(1024), (1 << 20) + 1, fake, None) == kivi.KIVI_EINVAL
    for code in (0, -1, -2, -3, -4, 7):
        assert isinstance(L.kivi_strerror(code), bytes)


def test_misaligned_pointers_are_rejected_before_any_launch():
    """16-byte alignment for the vector-loaded buffers, 4 bytes for the
    32-bit arrays and the fp32 output.  A decode call whose pointers pass
    and whose workspace is one byte short returns KIVI_ENOSPC, still before
    any launch, which tells the two checks apart."""
    L = kivi.lib()
    d = kivi.make_dims(2, 2, 128, 2, 32, 32, 256)
    need = kivi.workspace_bytes(d)
    p = ctypes.c_void_p
    fields = [n for n, _ in kivi.CacheStruct._fields_]
    four = {"q_len", "r_len", "status", "tickets"}

    def decode(cs, q=0x1000, out=0x1000, ws=0x1000):
        return L.kivi_decode_attn(ctypes.byref(d), ctypes.byref(cs), p(q), p(out),
                                  ctypes.c_float(1.0), p(ws), ctypes.c_size_t(need - 1), None)

    good = kivi.CacheStruct(*([0x1000] * len(fields)))
    assert decode(good) == kivi.KIVI_ENOSPC
    for name in fields:
        for addr in (0x1008, 0x1004, 0x1002):
            cs = kivi.CacheStruct(*([0x1000] * len(fields)))
            setattr(cs, name, addr)
            ok = name in four and addr % 4 == 0
            assert decode(cs) == (kivi.KIVI_ENOSPC if ok else kivi.KIVI_EINVAL), (name, addr)
            if not ok:
                assert L.kivi_flush_residual(ctypes.byref(d), ctypes.byref(cs), None) == \
                    kivi.KIVI_EINVAL
    assert decode(good, q=0x1008) == kivi.KIVI_EINVAL
    assert decode(good, ws=0x1008) == kivi.KIVI_EINVAL
    assert decode(good, out=0x1004) == kivi.KIVI_ENOSPC
    assert decode(good, out=0x1002) == kivi.KIVI_EINVAL
    f, m = p(0x1000), p(0x1008)
    assert L.kivi_append_kv(ctypes.byref(d), ctypes.byref(good), m, f, None) == kivi.KIVI_EINVAL
    assert L.kivi_append_kv(ctypes.byref(d), ctypes.byref(good), f, m, None) == kivi.KIVI_EINVAL
    assert L.kivi_prefill(ctypes.byref(d), ctypes.byref(good), m, f, 64, f, None, None) == \
        kivi.KIVI_EINVAL
    assert L.kivi_prefill(ctypes.byref(d), ctypes.byref(good), f, f, 64, p(0x1002), None, None) == \
        kivi.KIVI_EINVAL
    assert L.kivi_prefill(ctypes.byref(d), ctypes.byref(good), f, f, 64, f, p(0x1001), None) == \
        kivi.KIVI_EINVAL
    assert L.kivi_decode_step(ctypes.byref(d), ctypes.byref(good), m, f, f, f, ctypes.c_float(1.0),
                              f, ctypes.c_size_t(need), None) == kivi.KIVI_EINVAL
    assert L.kivi_decode_attn_sink(ctypes.byref(d), ctypes.byref(good), m, f, 4, f, f,
                                   ctypes.c_float(1.0), ctypes.c_double(0.0), f,
                                   ctypes.c_size_t(need), None) == kivi.KIVI_EINVAL
    for n, ks in ((-1, f), (4097, f), (4, None), (4, m)):
        assert L.kivi_decode_step_sink(ctypes.byref(d), ctypes.byref(good), f, f, ks, f, n, f, f,
                                       ctypes.c_float(1.0), f, ctypes.c_size_t(need),
                                       None) == kivi.KIVI_EINVAL
    assert L.kivi_decode_step_sink(ctypes.byref(d), ctypes.byref(good), f, f, None, None, 0, f, f,
                                   ctypes.c_float(1.0), f, ctypes.c_size_t(need - 1),
                                   None) == kivi.KIVI_ENOSPC
    # with no sink tokens the sink pointers are not read
    assert L.kivi_decode_attn_sink(ctypes.byref(d), ctypes.byref(good), m, None, 0, f, f,
                                   ctypes.c_float(1.0), ctypes.c_double(0.0), f,
                                   ctypes.c_size_t(need - 1), None) == kivi.KIVI_ENOSPC
    assert L.kivi_decode_attn_rope(ctypes.byref(d), ctypes.byref(good), m, f, ctypes.c_float(1.0),
                                   ctypes.c_double(1e4), f, ctypes.c_size_t(need),
                                   None) == kivi.KIVI_EINVAL
