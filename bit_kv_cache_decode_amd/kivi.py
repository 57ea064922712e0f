"""Python binding of libkivi (argument marshalling only).

Every step of the path runs in the HIP library; this module checks tensor
shapes, dtypes, devices and contiguity, passes raw device pointers and the
current HIP stream through the C ABI declared in ``include/kivi.h``, and turns
error codes into exceptions.  PyTorch provides device memory and streams.

If ``libkivi.so`` has not been built, every entry point raises: there is no
fallback implementation.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkivi.so")

KIVI_OK, KIVI_EINVAL, KIVI_ENOSPC, KIVI_EHIP, KIVI_EUNSUPPORTED = 0, -1, -2, -3, -4
ST_RESIDUAL_FULL, ST_CAPACITY, ST_BAD_LENGTH, ST_TICKETS = 0x1, 0x2, 0x4, 0x8

# Every symbol the public header declares.
EXPORTS = ("kivi_validate_dims", "kivi_cache_init", "kivi_workspace_init", "kivi_append_kv", "kivi_flush_residual", "kivi_prefill",
           "kivi_decode_workspace_bytes", "kivi_decode_splits", "kivi_decode_step_kernels", "kivi_decode_attn",
           "kivi_decode_attn_noalloc", "kivi_prefill_vq", "kivi_append_kv_vq",
           "kivi_flush_residual_vq", "kivi_decode_attn_vq",
           "kivi_decode_attn_rope", "kivi_decode_attn_sink", "kivi_decode_step",
           "kivi_decode_step_sink", "kivi_stream_read",
           "kivi_strerror")


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "heads", "head_dim", "bits", "group", "residual", "capacity")]


class CacheStruct(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "k_res", "v_res",
                 "q_len", "r_len", "status", "tickets")]


class KiviError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: {lib().kivi_strerror(code).decode()} ({code})")
        self.code = code


_LIB = None


def lib():
    """Load libkivi.so (once).  Raises if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bit_kv_cache_decode_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, V, I32 = ctypes.POINTER, ctypes.c_void_p, ctypes.c_int32
        L.kivi_validate_dims.argtypes = [P(Dims)]
        L.kivi_cache_init.argtypes = [P(Dims), P(CacheStruct), V]
        L.kivi_workspace_init.argtypes = [P(Dims), V, ctypes.c_size_t, V]
        L.kivi_append_kv.argtypes = [P(Dims), P(CacheStruct), V, V, V]
        L.kivi_flush_residual.argtypes = [P(Dims), P(CacheStruct), V]
        L.kivi_prefill.argtypes = [P(Dims), P(CacheStruct), V, V, I32, V, V, V]
        L.kivi_prefill_vq.argtypes = [P(Dims), P(CacheStruct), V, V, I32, V, V, V]
        L.kivi_append_kv_vq.argtypes = [P(Dims), P(CacheStruct), V, V, V]
        L.kivi_flush_residual_vq.argtypes = [P(Dims), P(CacheStruct), V]
        L.kivi_decode_attn_vq.argtypes = [P(Dims), P(CacheStruct), V, V, ctypes.c_float, V,
                                          ctypes.c_size_t, V]
        L.kivi_decode_workspace_bytes.argtypes = [P(Dims)]
        L.kivi_decode_workspace_bytes.restype = ctypes.c_size_t
        L.kivi_decode_splits.argtypes = [P(Dims)]
        L.kivi_decode_step_kernels.argtypes = [P(Dims)]
        L.kivi_decode_attn.argtypes = [P(Dims), P(CacheStruct), V, V, ctypes.c_float, V,
                                       ctypes.c_size_t, V]
        L.kivi_decode_attn_noalloc.argtypes = [P(Dims), P(CacheStruct), V, V, ctypes.c_float, V]
        L.kivi_decode_attn_rope.argtypes = [P(Dims), P(CacheStruct), V, V, ctypes.c_float,
                                            ctypes.c_double, V, ctypes.c_size_t, V]
        L.kivi_decode_attn_sink.argtypes = [P(Dims), P(CacheStruct), V, V, I32, V, V,
                                            ctypes.c_float, ctypes.c_double, V, ctypes.c_size_t,
                                            V]
        L.kivi_decode_step.argtypes = [P(Dims), P(CacheStruct), V, V, V, V, ctypes.c_float, V,
                                       ctypes.c_size_t, V]
        L.kivi_decode_step_sink.argtypes = [P(Dims), P(CacheStruct), V, V, V, V, I32, V, V,
                                            ctypes.c_float, V, ctypes.c_size_t, V]
        L.kivi_stream_read.argtypes = [V, ctypes.c_size_t, I32, V, V]
        L.kivi_strerror.argtypes = [ctypes.c_int]
        L.kivi_strerror.restype = ctypes.c_char_p
        for name in EXPORTS:
            # without declared argument types ctypes would pass 64-bit
            # pointers as 32-bit C ints
            if getattr(L, name).argtypes is None:
                raise RuntimeError(f"{name}: no argument types declared")
            if name not in ("kivi_decode_workspace_bytes", "kivi_strerror"):
                getattr(L, name).restype = ctypes.c_int
        _LIB = L
    return _LIB


def _check(rc, what):
    if rc != KIVI_OK:
        raise KiviError(rc, what)


def make_dims(batch, heads, head_dim, bits, group, residual, capacity):
    return Dims(batch, heads, head_dim, bits, group, residual, capacity)


def validate_dims(dims):
    return lib().kivi_validate_dims(ctypes.byref(dims))


def workspace_bytes(dims):
    return lib().kivi_decode_workspace_bytes(ctypes.byref(dims))


def decode_splits(dims):
    return lib().kivi_decode_splits(ctypes.byref(dims))


def decode_step_kernels(dims):
    return lib().kivi_decode_step_kernels(ctypes.byref(dims))


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, shape, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class KiviCache:
    """Device buffers of one quantized KV cache, in the layouts of kivi.h.

    Codes are stored as int32 tensors holding the uint32 words bit for bit.
    """

    def __init__(self, batch, heads, head_dim, bits, group, residual, capacity, device="cuda"):
        self.dims = make_dims(batch, heads, head_dim, bits, group, residual, capacity)
        rc = validate_dims(self.dims)
        _check(rc, "cache dims")
        D, G, R, cap = head_dim, group, residual, capacity
        W = D * bits // 32
        dev = torch.device(device)
        f16, i32 = torch.float16, torch.int32
        self.k_codes = torch.zeros((batch, heads, cap // G, W, G), dtype=i32, device=dev)
        self.v_codes = torch.zeros((batch, heads, cap // G, W, G), dtype=i32, device=dev)
        self.k_scale = torch.zeros((batch, heads, cap // G, D), dtype=f16, device=dev)
        self.k_zero = torch.zeros((batch, heads, cap // G, D), dtype=f16, device=dev)
        self.v_scale = torch.zeros((batch, heads, cap // G, D // G, G), dtype=f16, device=dev)
        self.v_zero = torch.zeros((batch, heads, cap // G, D // G, G), dtype=f16, device=dev)
        self.k_res = torch.zeros((batch, heads, R, D), dtype=f16, device=dev)
        self.v_res = torch.zeros((batch, heads, R, D), dtype=f16, device=dev)
        self.q_len = torch.zeros((batch,), dtype=i32, device=dev)
        self.r_len = torch.zeros((batch,), dtype=i32, device=dev)
        self.status = torch.zeros((1,), dtype=i32, device=dev)
        self.tickets = torch.zeros((batch, 64), dtype=i32, device=dev)
        self.workspace = None
        self._struct = None

    # -- convenience
    @property
    def shape(self):
        d = self.dims
        return dict(batch=d.batch, heads=d.heads, head_dim=d.head_dim, bits=d.bits,
                    group=d.group, residual=d.residual, capacity=d.capacity)

    def buffers(self):
        return {n: getattr(self, n) for n, _ in CacheStruct._fields_}

    def struct(self):
        if self._struct is None:
            self._struct = CacheStruct(*[getattr(self, n).data_ptr() for n, _ in CacheStruct._fields_])
        return self._struct

    def status_bits(self):
        return int(self.status.item()) & 0xFFFFFFFF

    def clear_status(self):
        self.status.zero_()

    def nbytes(self):
        return sum(t.numel() * t.element_size() for t in self.buffers().values())


def cache_init(cache):
    """kivi_cache_init: empty the cache (lengths, ticket counters, status)."""
    d = cache.dims
    _check(lib().kivi_cache_init(ctypes.byref(d), ctypes.byref(cache.struct()), _stream()),
           "kivi_cache_init")


def workspace_init(dims, workspace):
    """kivi_workspace_init: zero the split-merge counters of a workspace."""
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" \
            or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    _check(lib().kivi_workspace_init(ctypes.byref(dims), workspace.data_ptr(),
                                     ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                                     _stream()), "kivi_workspace_init")


def append_kv(cache, k_new, v_new):
    d = cache.dims
    _need(k_new, torch.float16, (d.batch, d.heads, d.head_dim), "k_new")
    _need(v_new, torch.float16, (d.batch, d.heads, d.head_dim), "v_new")
    _check(lib().kivi_append_kv(ctypes.byref(d), ctypes.byref(cache.struct()),
                                k_new.data_ptr(), v_new.data_ptr(), _stream()), "kivi_append_kv")


def flush_residual(cache):
    d = cache.dims
    _check(lib().kivi_flush_residual(ctypes.byref(d), ctypes.byref(cache.struct()), _stream()),
           "kivi_flush_residual")


def prefill(cache, k, v, lengths, window=None):
    """k, v: fp16 [batch, heads, src_len, head_dim]; lengths (and window, or
    None for lengths % G): int32 [batch] device tensors."""
    d = cache.dims
    src_len = k.shape[2]
    _need(k, torch.float16, (d.batch, d.heads, src_len, d.head_dim), "k")
    _need(v, torch.float16, (d.batch, d.heads, src_len, d.head_dim), "v")
    _need(lengths, torch.int32, (d.batch,), "lengths")
    if window is not None:
        _need(window, torch.int32, (d.batch,), "window")
    _check(lib().kivi_prefill(ctypes.byref(d), ctypes.byref(cache.struct()), k.data_ptr(),
                              v.data_ptr(), int(src_len), lengths.data_ptr(),
                              None if window is None else window.data_ptr(), _stream()),
           "kivi_prefill")


# ---- value queue: a cache kept with these four calls holds its values in
# an fp16 ring of the newest R, the older ones quantized token by token

def prefill_vq(cache, k, v, lengths, window=None):
    """kivi_prefill_vq: prefill with a value queue (arguments as prefill)."""
    d = cache.dims
    src_len = k.shape[2]
    _need(k, torch.float16, (d.batch, d.heads, src_len, d.head_dim), "k")
    _need(v, torch.float16, (d.batch, d.heads, src_len, d.head_dim), "v")
    _need(lengths, torch.int32, (d.batch,), "lengths")
    if window is not None:
        _need(window, torch.int32, (d.batch,), "window")
    _check(lib().kivi_prefill_vq(ctypes.byref(d), ctypes.byref(cache.struct()), k.data_ptr(),
                                 v.data_ptr(), int(src_len), lengths.data_ptr(),
                                 None if window is None else window.data_ptr(), _stream()),
           "kivi_prefill_vq")


def append_kv_vq(cache, k_new, v_new):
    d = cache.dims
    _need(k_new, torch.float16, (d.batch, d.heads, d.head_dim), "k_new")
    _need(v_new, torch.float16, (d.batch, d.heads, d.head_dim), "v_new")
    _check(lib().kivi_append_kv_vq(ctypes.byref(d), ctypes.byref(cache.struct()),
                                   k_new.data_ptr(), v_new.data_ptr(), _stream()),
           "kivi_append_kv_vq")


def flush_residual_vq(cache):
    d = cache.dims
    _check(lib().kivi_flush_residual_vq(ctypes.byref(d), ctypes.byref(cache.struct()), _stream()),
           "kivi_flush_residual_vq")


def decode_attn_vq(cache, q, sm_scale, out=None, workspace=None):
    """decode_attn over a value-queue cache; fp32 output."""
    d = cache.dims
    out, workspace, nbytes = _decode_buffers(cache, q, out, workspace)
    _check(lib().kivi_decode_attn_vq(ctypes.byref(d), ctypes.byref(cache.struct()), q.data_ptr(),
                                     out.data_ptr(), ctypes.c_float(sm_scale), workspace.data_ptr(),
                                     ctypes.c_size_t(nbytes), _stream()), "kivi_decode_attn_vq")
    return out


def new_workspace(dims, device="cuda"):
    """A zero-filled workspace of the size kivi_decode_attn needs."""
    n = workspace_bytes(dims)
    if n == 0:
        raise KiviError(KIVI_EINVAL, "kivi_decode_workspace_bytes")
    return torch.zeros((n,), dtype=torch.uint8, device=device)


def _decode_buffers(cache, q, out, workspace):
    d = cache.dims
    _need(q, torch.float16, (d.batch, d.heads, d.head_dim), "q")
    if out is None:
        out = torch.empty((d.batch, d.heads, d.head_dim), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, (d.batch, d.heads, d.head_dim), "out")
    if workspace is None:
        if cache.workspace is None:
            cache.workspace = new_workspace(d, q.device)
        workspace = cache.workspace
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return out, workspace, workspace.numel() * workspace.element_size()


def decode_attn(cache, q, sm_scale, out=None, workspace=None):
    """out[b, h] = softmax(sm_scale * q[b, h] . K^T) V over the cache; fp32."""
    d = cache.dims
    out, workspace, nbytes = _decode_buffers(cache, q, out, workspace)
    _check(lib().kivi_decode_attn(ctypes.byref(d), ctypes.byref(cache.struct()), q.data_ptr(),
                                  out.data_ptr(), ctypes.c_float(sm_scale), workspace.data_ptr(),
                                  ctypes.c_size_t(nbytes), _stream()), "kivi_decode_attn")
    return out


def decode_attn_noalloc(cache, q, sm_scale, out):
    """kivi_decode_attn_noalloc: decode_attn with the library's own device
    array as scratch (nothing is allocated; `out` is required)."""
    d = cache.dims
    _need(q, torch.float16, (d.batch, d.heads, d.head_dim), "q")
    _need(out, torch.float32, (d.batch, d.heads, d.head_dim), "out")
    _check(lib().kivi_decode_attn_noalloc(ctypes.byref(d), ctypes.byref(cache.struct()),
                                          q.data_ptr(), out.data_ptr(), ctypes.c_float(sm_scale),
                                          _stream()), "kivi_decode_attn_noalloc")
    return out


def decode_attn_rope(cache, q, sm_scale, rope_base=10000.0, out=None, workspace=None):
    """decode_attn with the cache's keys stored before the rotary embedding:
    each key is rotated by its position after dequantization; q is the
    already rotated query.  fp32 output."""
    d = cache.dims
    out, workspace, nbytes = _decode_buffers(cache, q, out, workspace)
    _check(lib().kivi_decode_attn_rope(ctypes.byref(d), ctypes.byref(cache.struct()), q.data_ptr(),
                                       out.data_ptr(), ctypes.c_float(sm_scale),
                                       ctypes.c_double(rope_base), workspace.data_ptr(),
                                       ctypes.c_size_t(nbytes), _stream()), "kivi_decode_attn_rope")
    return out


def decode_attn_sink(cache, q, sm_scale, k_sink, v_sink, rope_base=0.0, out=None,
                     workspace=None):
    """decode_attn over fp16 sink tokens (k_sink, v_sink: fp16
    [batch, heads, n_sink, head_dim]) followed by the cache's tokens; with
    rope_base > 1, keys (the sink's too) are stored before the rotary
    embedding and rotated by their positions (sink first); fp32 output."""
    d = cache.dims
    n_sink = k_sink.shape[2] if k_sink.dim() == 4 else -1
    _need(k_sink, torch.float16, (d.batch, d.heads, n_sink, d.head_dim), "k_sink")
    _need(v_sink, torch.float16, (d.batch, d.heads, n_sink, d.head_dim), "v_sink")
    out, workspace, nbytes = _decode_buffers(cache, q, out, workspace)
    _check(lib().kivi_decode_attn_sink(ctypes.byref(d), ctypes.byref(cache.struct()),
                                       k_sink.data_ptr(), v_sink.data_ptr(), ctypes.c_int32(n_sink),
                                       q.data_ptr(), out.data_ptr(), ctypes.c_float(sm_scale),
                                       ctypes.c_double(rope_base), workspace.data_ptr(),
                                       ctypes.c_size_t(nbytes), _stream()),
           "kivi_decode_attn_sink")
    return out


def decode_step_sink(cache, k_new, v_new, q, sm_scale, k_sink, v_sink, out=None,
                     workspace=None):
    """decode_step whose decode runs over fp16 sink tokens (k_sink, v_sink:
    fp16 [batch, heads, n_sink, head_dim]) followed by the cache's tokens."""
    d = cache.dims
    _need(k_new, torch.float16, (d.batch, d.heads, d.head_dim), "k_new")
    _need(v_new, torch.float16, (d.batch, d.heads, d.head_dim), "v_new")
    n_sink = k_sink.shape[2] if k_sink.dim() == 4 else -1
    _need(k_sink, torch.float16, (d.batch, d.heads, n_sink, d.head_dim), "k_sink")
    _need(v_sink, torch.float16, (d.batch, d.heads, n_sink, d.head_dim), "v_sink")
    out, workspace, nbytes = _decode_buffers(cache, q, out, workspace)
    _check(lib().kivi_decode_step_sink(ctypes.byref(d), ctypes.byref(cache.struct()),
                                       k_new.data_ptr(), v_new.data_ptr(), k_sink.data_ptr(),
                                       v_sink.data_ptr(), ctypes.c_int32(n_sink), q.data_ptr(),
                                       out.data_ptr(), ctypes.c_float(sm_scale),
                                       workspace.data_ptr(), ctypes.c_size_t(nbytes), _stream()),
           "kivi_decode_step_sink")
    return out


def decode_step(cache, k_new, v_new, q, sm_scale, out=None, workspace=None):
    """append_kv, decode_attn, flush_residual in one call (one kernel when a
    workgroup covers a whole (sequence, head)); returns the fp32 output."""
    d = cache.dims
    _need(k_new, torch.float16, (d.batch, d.heads, d.head_dim), "k_new")
    _need(v_new, torch.float16, (d.batch, d.heads, d.head_dim), "v_new")
    out, workspace, nbytes = _decode_buffers(cache, q, out, workspace)
    _check(lib().kivi_decode_step(ctypes.byref(d), ctypes.byref(cache.struct()), k_new.data_ptr(),
                                  v_new.data_ptr(), q.data_ptr(), out.data_ptr(),
                                  ctypes.c_float(sm_scale), workspace.data_ptr(),
                                  ctypes.c_size_t(nbytes), _stream()), "kivi_decode_step")
    return out


def stream_read(src, workgroups, sink=None):
    """Read the contiguous GPU tensor `src` once (kivi_stream_read, a
    measurement aid); returns the sink tensor (int32 [workgroups * 8])."""
    if not isinstance(src, torch.Tensor) or src.device.type != "cuda" or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    if sink is None:
        sink = torch.empty((workgroups * 8,), dtype=torch.int32, device=src.device)
    _need(sink, torch.int32, (workgroups * 8,), "sink")
    _check(lib().kivi_stream_read(src.data_ptr(), ctypes.c_size_t(src.numel() * src.element_size()),
                                  int(workgroups), sink.data_ptr(), _stream()), "kivi_stream_read")
    return sink
