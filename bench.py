#!/usr/bin/env python3
"""Benchmark of the quantized-KV decode hot path on one MI355X.

One step = the whole hot path for one batch: append the new token of every
(sequence, head) to the fp16 window, decode attention over the full context,
flush the now-full window into 2-bit codes -- one kivi_decode_step call (a
single kernel when one workgroup covers a whole (sequence, head)).  Default workload: the
Llama-2-7B-shaped layer (batch 8, 32 heads, head_dim 128, 3968 quantized +
128 window tokens at decode time, B=2, G=32, R=128), synthetic seeded data.

Each timed step runs on its own copy of the cache, all copies in the same
starting state (3968 quantized + 127 window tokens), so no step re-reads data
another step left in the 256 MB Infinity Cache.  The K timed steps are
captured in one HIP graph and replayed once between two synchronisations
(throughput); the same K steps are then launched eagerly from the same
starting state as separate calls, one phase at a time (all appends, all
decodes, all flushes), each phase a HIP graph replayed between HIP events on
the launch stream, which give the per-kernel average GPU durations of the
three separate kernels (the decode kernel's feeds the roofline); they must
leave the cache exactly as the whole-step kernel does, and give its output up
to rounding.  The decode of every other workload (the tiny, 13B, ragged
batch-64 and 131072-token ones, the last at B=2 and B=4) is then timed the
same way on rotated cache copies, with the 13B layer's full-window flush
timed separately, each beside its stream-read ceiling.  The CPU oracle is
timed beside it on bounded samples of (sequence, head) steps and decodes of
every workload.

Prints one JSON line on stdout; diagnostics go to stderr.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attn query-heads/sec over 2-bit KV; achieved HBM GB/s vs peak"
PEAK_HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
COPY_BUDGET_BYTES = 48e9
KERNEL_SRC = os.path.join(ROOT, "bit_kv_cache_decode_amd", "csrc", "kivi_kernels.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", type=int, default=2, help="workload number (1-5)")
    p.add_argument("--bits", type=int, default=None)
    p.add_argument("--cpu-seconds", type=float, default=8.0,
                   help="budget of the CPU oracle's whole-step sample")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--eager", action="store_true", help="launch steps eagerly instead of a graph")
    p.add_argument("--rope", type=float, default=None, metavar="BASE",
                   help="keys stored before the rotary embedding: the decode is "
                        "kivi_decode_attn_rope with this base, the step its three calls")
    p.add_argument("--sink", type=int, default=0, metavar="N",
                   help="N fp16 attention-sink tokens ahead of the cache: the decode is "
                        "kivi_decode_attn_sink, the step kivi_decode_step_sink (one kernel "
                        "where one workgroup covers a (sequence, head), else three)")
    p.add_argument("--no-stream", action="store_true",
                   help="skip the stream-read ceiling (kivi_stream_read) measurement")
    p.add_argument("--no-extra", action="store_true",
                   help="time only the chosen workload, not the decode of every other one")
    p.add_argument("--extra-steps", type=int, default=20,
                   help="decode launches timed per additional workload")
    p.add_argument("--copy-mb", type=int, default=0,
                   help="after the run, copy a buffer of this many MiB once (a known-size "
                        "reference dispatch for scaling hardware byte counters)")
    return p.parse_args()


def kernel_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload_name, key="bytes_per_launch"):
    """Per-launch HBM bytes of the decode kernel (or, with key
    "step_bytes_per_launch", of the whole-step kernel) from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_hash() or t.get("workload") != workload_name:
        return None
    return t.get(key)


def step_tokens(w):
    """Starting window sizes and the token every step appends.  Where every
    sequence's window holds at least one token, the cache starts one token
    short (r_len - 1 window tokens) and the step appends that last token, so
    after the append the cache holds exactly the workload's tokens.  Otherwise
    (empty windows in the ragged workload) the cache starts with the
    workload's tokens and the step appends one more, drawn N(0, 1) from seed
    2000 + workload number; then every window must have room for it."""
    import numpy as np
    cfg = w.config
    nb = len(w.r_len)  # the sequences drawn (the whole batch in the bench)
    if np.all(w.r_len >= 1):
        last = w.lengths - 1
        b = np.arange(nb)
        return (w.r_len - 1).astype(np.int32), np.ascontiguousarray(w.k[b, :, last]), \
            np.ascontiguousarray(w.v[b, :, last])
    if np.any(w.r_len >= cfg.residual):
        raise SystemExit("a full window cannot take the appended token")
    rng = np.random.Generator(np.random.PCG64(2000 + cfg.number))
    shape = (nb, cfg.heads, cfg.head_dim)
    k_new = rng.standard_normal(shape, dtype=np.float32).astype(np.float16)
    v_new = rng.standard_normal(shape, dtype=np.float32).astype(np.float16)
    return w.r_len.astype(np.int32), k_new, v_new


def cpu_baseline(w, budget_s):
    """Time the CPU oracle on whole steps (append, decode, flush) of single
    (sequence, head) pairs of the same workload, cycling over the pairs until
    the budget of timed work is spent.  Each pair's starting state is built
    once, untimed; every timed step runs on a fresh copy of it."""
    import numpy as np

    from oracle import cache as ocache

    cfg = w.config
    G, B, R = cfg.group, w.bits, cfg.residual
    r_start, k_new, v_new = step_tokens(w)
    pairs = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    states = {}
    done, spent = 0, 0.0
    while spent < budget_s:
        b, h = pairs[done % len(pairs)]
        ql, r0 = int(w.q_len[b]), int(r_start[b])
        if (b, h) not in states:
            states[(b, h)] = ocache.head_state(w.k[b, h], w.v[b, h], ql, r0, G, B,
                                               cfg.capacity, R)
        st = {k: (v.copy() if isinstance(v, np.ndarray) else v)
              for k, v in states[(b, h)].items()}
        t0 = time.perf_counter()
        st["k_res"][r0] = k_new[b, h]                         # append
        st["v_res"][r0] = v_new[b, h]
        st["r_len"] = rl = r0 + 1
        ocache.decode_head(w.q[b, h], st, cfg.sm_scale, G, B)  # decode
        if rl == R:                                           # flush
            enc = ocache.encode_tokens(st["k_res"], st["v_res"], G, B)
            g0 = ql // G
            st["k_codes"][g0:g0 + R // G] = enc["k_codes"]
            st["v_codes"][g0:g0 + R // G] = enc["v_codes"]
        spent += time.perf_counter() - t0
        done += 1
    nt = blas_threads()
    return {"value": done / spent, "unit": "query-heads/s", "cores": nt or 1, "kind": "oracle",
            "sample": f"{done} (sequence, head) steps (append + decode + flush each) cycling "
                      f"over the {len(pairs)} pairs of the same workload, numpy with its BLAS "
                      f"threads at their default ({nt}), {spent:.1f} s of timed work",
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "blas_threads": nt}


def stream_ceiling(nbytes, steps):
    """The HBM read rate this device sustains for the decode's byte count:
    kivi_stream_read over buffers of nbytes (rounded up to 16), rotated among
    enough copies that none is re-read from the 256 MB Infinity Cache, timed
    like the other workloads (time_graph: a HIP graph of `steps` launches)
    at several grid sizes; the fastest grid gives the ceiling."""
    import torch
    from bit_kv_cache_decode_amd import kivi

    n16 = (int(nbytes) + 15) // 16
    n_rot = min(64, max(2, -(-int(ROTATE_BYTES) // (n16 * 16))))
    bufs = [torch.full((n16 * 4,), i + 1, dtype=torch.int32, device="cuda") for i in range(n_rot)]
    by_wg = {}
    for wg in (256, 512, 1024, 2048):
        sink = torch.empty((wg * 8,), dtype=torch.int32, device="cuda")
        by_wg[wg] = time_graph(lambda i: kivi.stream_read(bufs[i % n_rot], wg, sink), steps)
        del sink
    best = min(by_wg, key=by_wg.get)
    us = by_wg[best]
    del bufs
    torch.cuda.empty_cache()
    return {"kernel": "stream_read_kernel (kivi_stream_read)", "bytes": n16 * 16,
            "workgroups": best, "us": us, "GBps": n16 * 16 / (us * 1e-6) / 1e9,
            "frac_of_peak": n16 * 16 / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS,
            "us_by_workgroups": {str(k): round(v, 3) for k, v in by_wg.items()},
            "rotated_buffers": n_rot}


# The other workloads' decodes, each timed beside the headline one: (workload
# number, B) in the order they run.  The long-context draws serve B=2 and
# B=4 (the same fp16 tokens, quantized at either width).
EXTRA_WORKLOADS = ((1, None), (3, None), (4, None), (5, 2), (5, 4))
ROTATE_BYTES = 1.2e9


def warm_gpu(replay, warm_ms):
    """Run ``replay`` (one graph replay) until ``warm_ms`` of GPU time has
    passed (at least twice)."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    replay()
    e1.record()
    torch.cuda.synchronize()
    one = max(e0.elapsed_time(e1), 1e-3)
    for _ in range(max(1, int(warm_ms / one))):
        replay()
    torch.cuda.synchronize()


def time_graph(fn, n, reps=3, warm_ms=20.0):
    """HIP graph of fn(0) .. fn(n - 1), replayed for at least ``warm_ms`` of
    GPU time to warm up, then ``reps`` times between HIP events on the
    launch stream; the median, in microseconds per call.  (Right after a
    large workload's host-side set-up the GPU runs its first milliseconds
    of work 10-20% slower than later ones.)"""
    import numpy as np
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    warm_gpu(g.replay, warm_ms)
    times = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(1e3 * e0.elapsed_time(e1) / n)
    return float(np.median(times))


def measure_workload(w, steps, no_stream):
    """Decode of workload ``w`` at its own lengths (and, where every window
    is full, the flush of those windows), timed over ``steps`` launches
    rotated over cache copies that together exceed the 256 MB Infinity
    Cache several times; the rate against 8 TB/s and against the stream-read
    ceiling at the same byte count."""
    import torch
    from bit_kv_cache_decode_amd import kivi
    from bit_kv_cache_decode_amd import workloads as wl

    cfg = w.config
    dims = w.dims()
    Bt, H, D = dims["batch"], cfg.heads, cfg.head_dim
    base = kivi.KiviCache(**dims)
    kt = torch.from_numpy(w.k).cuda()
    vt = torch.from_numpy(w.v).cuda()
    q0 = torch.from_numpy(w.q_len).cuda()
    r0 = torch.from_numpy(w.r_len).cuda()
    kivi.prefill(base, kt, vt, q0 + r0, r0)
    del kt, vt
    q = torch.from_numpy(w.q).cuda()
    torch.cuda.synchronize()
    assert base.status_bits() == 0
    cb = base.nbytes()
    n = int(max(1, min(steps, max(2, -(-ROTATE_BYTES // cb)), COPY_BUDGET_BYTES // cb)))
    copies = [base]
    for _ in range(n - 1):
        c = kivi.KiviCache(**dims)
        for name, t in base.buffers().items():
            getattr(c, name).copy_(t)
        copies.append(c)
    outs = [torch.empty((Bt, H, D), dtype=torch.float32, device="cuda") for _ in range(n)]
    ws = kivi.new_workspace(base.dims)
    us = time_graph(lambda i: kivi.decode_attn(copies[i % n], q, cfg.sm_scale, out=outs[i % n],
                                               workspace=ws), steps)
    ok = all(c.status_bits() == 0 for c in copies)
    nbytes = int(wl.decode_bytes(w.q_len, w.r_len, H, D, w.bits, cfg.group))
    gbps = nbytes / (us * 1e-6) / 1e9
    res = {"workload": cfg.name + (f" at B={w.bits}" if w.bits != cfg.bits else ""),
           "description": cfg.description, "batch": Bt, "heads": H, "bits": w.bits,
           "group": cfg.group, "quantized_tokens": int(w.q_len.sum()),
           "window_tokens": int(w.r_len.sum()), "splits": kivi.decode_splits(base.dims),
           "decode_us": us, "algorithmic_bytes": nbytes, "GBps": gbps,
           "frac": gbps / PEAK_HBM_GBPS, "query_heads_per_s": Bt * H / (us * 1e-6),
           "launches": steps, "cache_copies": n, "status_clean": ok}
    if bool((w.r_len == cfg.residual).all()):
        # every window is full: the flush of all of them, each launch on a
        # fresh copy (the lengths put back between the warm-up and the timed
        # replay)
        nf = min(steps, n)

        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(nf):
                kivi.flush_residual(copies[i])
        times = []
        for _ in range(5):  # two warm-up replays, then the median of three
            for c in copies[:nf]:
                c.q_len.copy_(q0)
                c.r_len.copy_(r0)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(1e3 * e0.elapsed_time(e1) / nf)
        fus = float(sorted(times[2:])[1])
        fb = Bt * H * wl.flush_bytes_per_head(cfg.residual, D, w.bits, cfg.group)
        res["flush"] = {"us": fus, "windows": Bt * H, "algorithmic_bytes": int(fb),
                        "GBps": fb / (fus * 1e-6) / 1e9,
                        "frac": fb / (fus * 1e-6) / 1e9 / PEAK_HBM_GBPS, "launches": nf,
                        "committed": bool(all(int(c.q_len[0]) == int(w.q_len[0]) + cfg.residual
                                              for c in copies[:nf]))}
    del copies, outs, ws, base
    torch.cuda.empty_cache()
    if not no_stream:
        sr = stream_ceiling(nbytes, steps)
        res["stream_read_us"] = sr["us"]
        res["stream_read_frac"] = sr["frac_of_peak"]
        res["decode_frac_of_stream_read"] = gbps / sr["GBps"]
    return res


def oracle_sample(w, n_heads, seed, flush=False):
    """Wall time of the CPU oracle's decode (dequantization plus fp64
    attention) on ``n_heads`` (sequence, head) pairs of workload ``w`` drawn
    with ``seed`` (their cache states are encoded beforehand, untimed), and,
    with ``flush``, of quantizing and packing their full windows; numpy with
    its BLAS threads at their default."""
    import numpy as np
    from oracle import cache as ocache

    cfg = w.config
    rng = np.random.default_rng(seed)
    nb = w.q.shape[0]
    pairs = [(int(b), int(h)) for b, h in zip(rng.integers(0, nb, n_heads),
                                              rng.integers(0, cfg.heads, n_heads))]
    states = [ocache.head_state(w.k[b, h], w.v[b, h], int(w.q_len[b]), int(w.r_len[b]),
                                cfg.group, w.bits, cfg.capacity, cfg.residual) for b, h in pairs]
    t0 = time.perf_counter()
    for (b, h), st in zip(pairs, states):
        ocache.decode_head(w.q[b, h], st, cfg.sm_scale, cfg.group, w.bits)
    dec = time.perf_counter() - t0
    out = {"heads": n_heads, "decode_s": dec, "query_heads_per_s": n_heads / dec}
    if flush:
        t0 = time.perf_counter()
        for st in states:
            ocache.encode_tokens(st["k_res"], st["v_res"], cfg.group, w.bits)
        fl = time.perf_counter() - t0
        out.update({"flush_s": fl, "flushes_per_s": n_heads / fl})
    return out


# (sequence, head) pairs the oracle decodes per workload for the CPU baseline
ORACLE_SAMPLE_HEADS = {1: 1, 2: 64, 3: 64, 4: 64, 5: 2}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 0) for i in threadpool_info()
                    if i.get("user_api") == "blas"), default=None)
    except Exception:
        return None


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log("bench.py measures one GPU only: this build has no multi-GPU path "
            "(decode shards by (sequence, head) with no communication).")
        sys.exit(2)

    import numpy as np
    import torch

    from bit_kv_cache_decode_amd import kivi
    from bit_kv_cache_decode_amd import workloads as wl

    torch.cuda.set_device(0)
    w = wl.generate(args.workload, bits=args.bits)
    cfg = w.config
    dims = w.dims()
    Bt, H, D = cfg.batch, cfg.heads, cfg.head_dim
    K, W = args.steps, args.warmup
    r_start, k_new, v_new = step_tokens(w)

    # ---- the starting state: q_len quantized + r_start window tokens
    kt = torch.from_numpy(w.k).cuda()
    vt = torch.from_numpy(w.v).cuda()
    base = kivi.KiviCache(**dims)
    q0 = torch.from_numpy(w.q_len).cuda()
    r0 = torch.from_numpy(r_start).cuda()
    kivi.prefill(base, kt, vt, q0 + r0, r0)
    k_new = torch.from_numpy(k_new).cuda()   # [batch, heads, D]
    v_new = torch.from_numpy(v_new).cuda()
    q = torch.from_numpy(w.q).cuda()
    k_sink, v_sink = (torch.from_numpy(x).cuda() for x in wl.sink_tokens(w, args.sink))
    del kt, vt
    torch.cuda.synchronize()
    assert base.status_bits() == 0

    # every timed step runs on its own copy of the starting state; the number
    # of copies (and so of timed steps) is capped by a memory budget
    cache_bytes = base.nbytes()
    max_copies = max(2, int(COPY_BUDGET_BYTES // cache_bytes))
    if max(K, W) > max_copies:
        log(f"{max(K, W)} steps need {max(K, W)} cache copies of {cache_bytes / 1e9:.2f} GB; "
            f"timing {min(K, max_copies)} steps, warming up {min(W, max_copies)}")
        K, W = min(K, max_copies), min(W, max_copies)
    n_copies = max(K, W)
    copies = [base]
    for _ in range(n_copies - 1):
        c = kivi.KiviCache(**dims)
        for name, t in base.buffers().items():
            getattr(c, name).copy_(t)
        copies.append(c)
    outs = [torch.empty((Bt, H, D), dtype=torch.float32, device="cuda") for _ in range(n_copies)]
    ws = kivi.new_workspace(base.dims)
    log(f"workload {cfg.name}: {n_copies} cache copies of {cache_bytes / 1e6:.1f} MB")

    def reset():
        for c in copies:
            c.q_len.copy_(q0)
            c.r_len.copy_(r0)

    def decode(i, out):
        if args.sink:
            return kivi.decode_attn_sink(copies[i], q, cfg.sm_scale, k_sink, v_sink,
                                         rope_base=args.rope or 0.0, out=out, workspace=ws)
        if args.rope is None:
            return kivi.decode_attn(copies[i], q, cfg.sm_scale, out=out, workspace=ws)
        return kivi.decode_attn_rope(copies[i], q, cfg.sm_scale, args.rope, out=out, workspace=ws)

    def step(i):
        # append + decode + flush: one kernel when one workgroup covers a
        # whole (sequence, head), else the three kernels (always three with
        # keys stored before the rotary embedding or with a sink)
        if args.rope is None and not args.sink:
            kivi.decode_step(copies[i], k_new, v_new, q, cfg.sm_scale, out=outs[i], workspace=ws)
        elif args.rope is None:
            kivi.decode_step_sink(copies[i], k_new, v_new, q, cfg.sm_scale, k_sink, v_sink,
                                  out=outs[i], workspace=ws)
        else:
            kivi.append_kv(copies[i], k_new, v_new)
            decode(i, outs[i])
            kivi.flush_residual(copies[i])

    # ---- warmup (eager), then back to the starting state
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    eager_out0 = outs[0].clone()
    reset()
    torch.cuda.synchronize()

    # The decode phase as a graph of its own, captured first: it reads the
    # caches and writes only the outputs, so replaying it warms the GPU
    # before each timed region without touching the cache state.
    dgraph = None
    if not args.eager:
        dgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(dgraph):
            for i in range(K):
                decode(i, outs[i])
        dgraph.replay()
        torch.cuda.synchronize()

    # ---- timed region 1: the K steps as one HIP graph, replayed once
    graph = None
    noflush_us = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(K):
                step(i)
        # one untimed replay first: a graph's first replay carries one-time
        # costs (its upload to the device) that would otherwise land in the
        # timed region
        graph.replay()
        torch.cuda.synchronize()
        reset()
        torch.cuda.synchronize()
        warm_gpu(dgraph.replay, 20.0)
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        g0.record()
        graph.replay()
        g1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        step_event_us = 1e3 * g0.elapsed_time(g1) / K
        replay_ok = bool(torch.equal(outs[0], eager_out0))
        states_ok = bool(all(c.status_bits() == 0 for c in copies[:K]))
        step_state = {n: t.clone() for n, t in copies[0].buffers().items()}
        reset()
        torch.cuda.synchronize()

    # ---- timed region 2: the same K steps one phase at a time (the K
    # appends, then the K decodes, then the K flushes; every copy is
    # independent, so the results are those of K whole steps), each phase a
    # HIP graph replayed once between HIP events on the launch stream: each
    # kernel's average duration is its phase time over K, with no host-side
    # launch cost in it (eager launches with --eager).
    phases = [
        lambda i: kivi.append_kv(copies[i], k_new, v_new),
        lambda i: decode(i, outs[i]),
        lambda i: kivi.flush_residual(copies[i]),
    ]
    pgraphs = []
    if not args.eager:
        for p_i, fn in enumerate(phases):
            if p_i == 1:
                pgraphs.append(dgraph)
                continue
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(K):
                    fn(i)
            pgraphs.append(g)
        for g in pgraphs:      # untimed first replays, in phase order
            g.replay()
        torch.cuda.synchronize()
        reset()
        torch.cuda.synchronize()
        # then 20 ms of the decode phase alone (it reads the caches and writes
        # only the outputs), so that the timed phases start on a warm GPU
        warm_gpu(pgraphs[1].replay, 20.0)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    t0 = time.perf_counter()
    evs[0].record()
    for p_i, fn in enumerate(phases):
        if pgraphs:
            pgraphs[p_i].replay()
        else:
            for i in range(K):
                fn(i)
        evs[p_i + 1].record()
    torch.cuda.synchronize()
    eager_wall = time.perf_counter() - t0
    if graph is None:
        wall = eager_wall
    # The three kernels must leave the cache bit for bit as the whole-step
    # kernel does; their output may differ from it by rounding only (the
    # whole-step kernel may take the window tokens first).
    # (up to rounding: the plain decode and the whole-step kernel sum in
    # different lane orders)
    eager_ok = bool(torch.allclose(outs[0], eager_out0, rtol=1e-4, atol=1e-4))
    if graph is None:
        replay_ok = eager_ok
        states_ok = bool(all(c.status_bits() == 0 for c in copies[:K]))
    else:
        eager_ok = eager_ok and all(torch.equal(t, step_state[n])
                                    for n, t in copies[0].buffers().items())

    append_us = 1e3 * evs[0].elapsed_time(evs[1]) / K
    decode_us = 1e3 * evs[1].elapsed_time(evs[2]) / K
    flush_us = 1e3 * evs[2].elapsed_time(evs[3]) / K
    if not (replay_ok and states_ok and eager_ok):
        log(f"WARNING: outputs match the warmup's: graph {replay_ok}, phased {eager_ok}; "
            f"status clean: {states_ok}")

    # ---- the whole-step graph again, from windows two tokens shorter: every
    # step appends and decodes without filling the window (the common step in
    # serving, where one step in R flushes); the copies' bytes are the same.
    # It writes window slots that the phased run above reads, so it comes
    # after that comparison.
    if graph is not None and bool((r0 >= 2).all()):
        for c in copies:
            c.q_len.copy_(q0)
            c.r_len.copy_(r0 - 2)
        torch.cuda.synchronize()
        warm_gpu(dgraph.replay, 20.0)
        g0.record()
        graph.replay()
        g1.record()
        torch.cuda.synchronize()
        noflush_us = 1e3 * g0.elapsed_time(g1) / K
        noflush_ok = bool(all(c.status_bits() == 0 for c in copies[:K])) and bool(
            (copies[0].r_len == r0 - 1).all())
        if not noflush_ok:
            log("WARNING: the non-flushing steps left an unexpected state")
        reset()
        torch.cuda.synchronize()

    # ---- per-call decode durations: HIP events around each of `calls`
    # separate launches, every copy back in the decode phase's state (its
    # starting lengths plus the appended token, which the window still holds)
    for c in copies:
        c.q_len.copy_(q0)
        c.r_len.copy_(r0 + 1)
    torch.cuda.synchronize()
    calls = max(200, K)
    pc = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(calls)]
    for i, (e0, e1) in enumerate(pc):
        e0.record()
        decode(i % n_copies, outs[i % n_copies])
        e1.record()
    torch.cuda.synchronize()
    per_call = np.array([1e3 * e0.elapsed_time(e1) for e0, e1 in pc])
    reset()
    torch.cuda.synchronize()

    step_s = wall / K
    plain = args.rope is None and not args.sink
    same_bits = w.bits == cfg.bits  # the counter runs are at the workload's own width
    one_kernel = kivi.decode_step_kernels(base.dims) == 1 and args.rope is None
    qheads = Bt * H
    dec_bytes = (wl.decode_bytes(w.q_len, r_start + 1, H, D, w.bits, cfg.group)
                 + Bt * H * args.sink * D * 2 * 2)   # fp16 sink keys and values
    achieved = dec_bytes / (decode_us * 1e-6) / 1e9
    n_flush = int((r_start + 1 == cfg.residual).sum()) * H
    flush_b = n_flush * wl.flush_bytes_per_head(cfg.residual, D, w.bits, cfg.group)
    result = {
        "metric": METRIC,
        "value": qheads / step_s,
        "unit": "query-heads/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.description}"
                        + (f", run at B={w.bits}" if w.bits != cfg.bits else ""),
            "batch": Bt, "heads": H, "head_dim": D, "bits": w.bits, "group": cfg.group,
            "residual": cfg.residual,
            "context": int((w.q_len + r_start + 1).max()),
            "quantized_tokens": int(w.q_len.max()), "window_tokens": int((r_start + 1).max()),
            "rope_base": args.rope, "sink_tokens": args.sink,
            "step": (("kivi_decode_step (append + decode + flush, " if plain else
                      "kivi_decode_step_sink (append + decode + flush, " if args.rope is None else
                      "kivi_append_kv + kivi_decode_attn_%s + kivi_flush_residual ("
                      % ("sink" if args.sink else "rope"))
                     + ("one kernel" if one_kernel else "three kernels")
                     + "), " + ("one HIP graph of all timed steps" if graph is not None
                                else "eager launches")),
        },
        "decode": {"us": decode_us, "query_heads_per_s": qheads / (decode_us * 1e-6),
                   "algorithmic_bytes": int(dec_bytes), "GBps": achieved},
        "decode_per_call_us": {"median": float(np.median(per_call)),
                               "p10": float(np.percentile(per_call, 10)),
                               "p90": float(np.percentile(per_call, 90)), "calls": calls},
        "phased_ms_per_step": eager_wall / K * 1e3,
        "append_us": append_us,
        "flush_us": flush_us,
        # the flush phase: the windows the appended token filled, quantized
        # (their algorithmic bytes over the phase's per-step time)
        "flush": {"us": flush_us, "windows": n_flush,
                  "algorithmic_bytes": int(flush_b),
                  "GBps": flush_b / (flush_us * 1e-6) / 1e9 if n_flush else 0.0,
                  "frac": flush_b / (flush_us * 1e-6) / 1e9 / PEAK_HBM_GBPS if n_flush else 0.0},
        "graph_replay_matches_eager": replay_ok,
        "phased_matches_step": eager_ok,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": measured_traffic(cfg.name) if plain and same_bits else None},
    }
    if one_kernel and graph is not None:
        # the whole-step kernel itself: the step's algorithmic bytes over its
        # per-step time inside the graph (HIP events around the replay)
        sb = (wl.step_bytes(w.q_len, r_start, H, D, w.bits, cfg.group, cfg.residual)
              + Bt * H * args.sink * D * 2 * 2)
        result["step_kernel"] = {
            "kernel": "decode_kernel whole-step variant (kivi_decode_step%s)"
                      % ("_sink" if args.sink else ""),
            "us": step_event_us, "algorithmic_bytes": sb,
            "GBps": sb / (step_event_us * 1e-6) / 1e9,
            "frac": sb / (step_event_us * 1e-6) / 1e9 / PEAK_HBM_GBPS,
            "traffic": (measured_traffic(cfg.name, "step_bytes_per_launch")
                        if plain and same_bits else None)}
        if noflush_us is not None:
            nb = (wl.step_bytes(w.q_len, r_start - 2, H, D, w.bits, cfg.group, cfg.residual)
                  + Bt * H * args.sink * D * 2 * 2)
            result["step_kernel_noflush"] = {
                "what": "the same whole-step kernel on windows two tokens short of full: "
                        "append and decode, no flush (the serving case)",
                "us": noflush_us, "query_heads_per_s": qheads / (noflush_us * 1e-6),
                "algorithmic_bytes": nb, "GBps": nb / (noflush_us * 1e-6) / 1e9,
                "frac": nb / (noflush_us * 1e-6) / 1e9 / PEAK_HBM_GBPS}
    if not args.no_stream:
        sr = stream_ceiling(dec_bytes, K)
        result["stream_read"] = sr
        result["decode_frac_of_stream_read"] = achieved / sr["GBps"]
    if args.copy_mb:
        # an elementwise kernel (not a DMA-engine memcpy, which no counter sees)
        src = torch.ones(args.copy_mb << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        result["copy_reference_bytes"] = int(src.numel() * 4)
    # ---- every other workload's decode (and the 13B layer's flush), on
    # the GPU and, as a baseline, the oracle on the host
    del graph, pgraphs, phases, copies, outs, base, ws
    torch.cuda.empty_cache()
    per_cpu = {}
    if not args.no_cpu:
        per_cpu[cfg.name] = oracle_sample(w, ORACLE_SAMPLE_HEADS[cfg.number], 7000 + cfg.number,
                                          flush=cfg.number == 3)
    extra = {}
    if not args.no_extra and args.rope is None and not args.sink:
        import dataclasses
        drawn = None
        for number, bits in EXTRA_WORKLOADS:
            if number == cfg.number and (bits or wl.CONFIGS[number].bits) == w.bits:
                continue
            if drawn is None or drawn.config.number != number:
                drawn = None
                drawn = wl.generate(number)
            we = drawn if bits is None else dataclasses.replace(drawn, bits=bits)
            log(f"workload {we.config.name} at B={we.bits}")
            r = measure_workload(we, args.extra_steps, args.no_stream)
            extra[r["workload"]] = r
            if not args.no_cpu:
                per_cpu[r["workload"]] = oracle_sample(we, ORACLE_SAMPLE_HEADS[number],
                                                       7000 + number, flush=number == 3)
        del drawn
        result["workloads"] = extra
    if not args.no_cpu:
        cb = cpu_baseline(w, args.cpu_seconds)
        cb["per_workload"] = per_cpu
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
