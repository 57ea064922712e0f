"""Shared helpers of the GPU parity tests (imported only by tests)."""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch
from threadpoolctl import threadpool_limits

from bit_kv_cache_decode_amd import kivi
from bit_kv_cache_decode_amd import workloads as wl
from oracle import cache as ocache

# Tolerance stated for the decode outputs against the fp64 oracle on the same
# dequantized values: max-abs error and relative L2 error.
MAX_ABS = 2e-3
REL_L2 = 1e-3

_WORKLOADS = {}


def workload(number, bits=None, batch=None):
    key = (number, bits, batch)
    if key not in _WORKLOADS:
        _WORKLOADS.clear()           # keep at most one large draw alive
        _WORKLOADS[key] = wl.generate(number, bits=bits, batch=batch)
    return _WORKLOADS[key]


def gpu_cache(w, capacity=None, q_len=None, r_len=None, residual=None):
    """Cache on the GPU holding the workload's tokens, built by kivi_prefill."""
    d = w.dims()
    if capacity is not None:
        d["capacity"] = capacity
    if residual is not None:
        d["residual"] = residual
    ql = w.q_len if q_len is None else np.asarray(q_len, np.int32)
    rl = w.r_len if r_len is None else np.asarray(r_len, np.int32)
    c = kivi.KiviCache(**d)
    k = torch.from_numpy(w.k).cuda()
    v = torch.from_numpy(w.v).cuda()
    lens = torch.from_numpy((ql + rl).astype(np.int32)).cuda()
    win = torch.from_numpy(rl.astype(np.int32)).cuda()
    kivi.prefill(c, k, v, lens, win)
    torch.cuda.synchronize()
    del k, v
    return c


def head_buffers(c, b, h):
    """One (sequence, head) of a GPU cache as numpy arrays (codes as uint32)."""
    out = {}
    for name in ("k_codes", "v_codes"):
        out[name] = getattr(c, name)[b, h].cpu().numpy().view(np.uint32)
    for name in ("k_scale", "k_zero", "v_scale", "v_zero", "k_res", "v_res"):
        out[name] = getattr(c, name)[b, h].cpu().numpy()
    out["q_len"] = int(c.q_len[b].item())
    out["r_len"] = int(c.r_len[b].item())
    return out


def oracle_head(w, b, h, capacity=None):
    cfg = w.config
    cap = cfg.capacity if capacity is None else capacity
    ql, rl = int(w.q_len[b]), int(w.r_len[b])
    return ocache.head_state(w.k[b, h], w.v[b, h], ql, rl, cfg.group, w.bits, cap, cfg.residual)


def assert_head_bit_exact(gpu, ref, group):
    ql, rl = ref["q_len"], ref["r_len"]
    assert gpu["q_len"] == ql and gpu["r_len"] == rl
    nt = ql // group
    for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
        g, r = gpu[name][:nt], ref[name][:nt]
        assert np.array_equal(g.view(np.uint8), r.view(np.uint8)), name
    for name in ("k_res", "v_res"):
        assert np.array_equal(gpu[name][:rl].view(np.uint8), ref[name][:rl].view(np.uint8)), name


def decode_errors(out, ref):
    """(max-abs error, relative L2 error) of fp32 outputs against fp64 ones."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    err = out - ref
    denom = np.linalg.norm(ref)
    return float(np.abs(err).max()), float(np.linalg.norm(err) / (denom if denom > 0 else 1.0))


def assert_within_tolerance(out, ref, label=""):
    mx, rel = decode_errors(out, ref)
    assert mx <= MAX_ABS and rel <= REL_L2, f"{label}: max-abs {mx:.3e}, rel-L2 {rel:.3e}"
    return mx, rel


def parallel_map(fn, items, workers=8):
    """fn over items on a pool of threads, numpy's BLAS held to one thread
    each (the oracle's array work releases the interpreter lock); returns the
    results in order."""
    with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, items))


def host_buffers(c):
    """Every buffer of a GPU cache as numpy arrays (codes as uint32)."""
    out = {n: t.cpu().numpy() for n, t in c.buffers().items()}
    for n in ("k_codes", "v_codes", "tickets", "status"):
        out[n] = out[n].view(np.uint32)
    return out


def head_of(buffers, b, h):
    """One (sequence, head) of host_buffers() in the head_buffers() form."""
    out = {n: buffers[n][b, h] for n in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale",
                                          "v_zero", "k_res", "v_res")}
    out["q_len"] = int(buffers["q_len"][b])
    out["r_len"] = int(buffers["r_len"][b])
    return out
