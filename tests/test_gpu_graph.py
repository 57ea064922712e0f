"""The library's calls under HIP graph capture: each captured call replayed
several times, with the program's own eager work and synchronisations
between the replays, gives exactly what the eager call gives (the kernels
are deterministic and record no memset nodes)."""

import numpy as np
import pytest
import torch

from bit_kv_cache_decode_amd import kivi
from bit_kv_cache_decode_amd import workloads as wl
from tests.gpu_common import gpu_cache, workload

pytestmark = pytest.mark.gpu


def _decodes(c, q, ks, vs, outs, ws):
    kivi.decode_attn(c, q, 1.0, out=outs[0], workspace=ws)
    kivi.decode_attn_rope(c, q, 1.0, 10000.0, out=outs[1], workspace=ws)
    kivi.decode_attn_sink(c, q, 1.0, ks, vs, out=outs[2], workspace=ws)
    kivi.decode_attn_sink(c, q, 1.0, ks, vs, rope_base=10000.0, out=outs[3], workspace=ws)


@pytest.mark.parametrize("capacity", [None, 65536])
def test_captured_decodes_replay_as_eager(capacity):
    """Plain, rotary, sink and rotary-sink decodes; one workgroup per
    (sequence, head), and several with a split merge (capacity 65536)."""
    w = workload(2, batch=2)
    c = gpu_cache(w, capacity=capacity)
    q = torch.from_numpy(w.q).cuda()
    ks, vs = (torch.from_numpy(x).cuda() for x in wl.sink_tokens(w, 8))
    ws = kivi.new_workspace(c.dims)
    outs = [torch.empty((2, 32, 128), dtype=torch.float32, device="cuda") for _ in range(4)]
    _decodes(c, q, ks, vs, outs, ws)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _decodes(c, q, ks, vs, outs, ws)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o, e), (rep, i)
        assert c.status_bits() == 0


def test_captured_whole_step_replays_as_eager():
    """kivi_decode_step (append, decode, flush in one kernel) and the three
    calls, captured; before each replay the cache is put back into its
    starting state eagerly, and every replay leaves the same cache state and
    output as the eager step."""
    w = workload(2)                                          # 8 x 32: one workgroup each
    d = w.dims()
    B = w.config.batch
    base = gpu_cache(w, q_len=w.q_len, r_len=w.r_len - 1)   # one token short
    last = w.lengths - 1
    k_new = torch.from_numpy(np.ascontiguousarray(w.k[np.arange(B), :, last])).cuda()
    v_new = torch.from_numpy(np.ascontiguousarray(w.v[np.arange(B), :, last])).cuda()
    q = torch.from_numpy(w.q).cuda()
    assert kivi.decode_step_kernels(base.dims) == 1
    work = [kivi.KiviCache(**d) for _ in range(2)]
    ws = kivi.new_workspace(base.dims)
    outs = [torch.empty((B, 32, 128), dtype=torch.float32, device="cuda") for _ in range(2)]

    def reset():
        for c in work:
            for name, t in base.buffers().items():
                getattr(c, name).copy_(t)

    def step():
        kivi.decode_step(work[0], k_new, v_new, q, 1.0, out=outs[0], workspace=ws)
        kivi.append_kv(work[1], k_new, v_new)
        kivi.decode_attn(work[1], q, 1.0, out=outs[1], workspace=ws)
        kivi.flush_residual(work[1])

    reset()
    step()
    torch.cuda.synchronize()
    eager_out = [o.clone() for o in outs]
    eager_state = [{n: t.clone() for n, t in c.buffers().items()} for c in work]
    assert int(work[0].r_len[0]) == 0                        # the step flushed
    g = torch.cuda.CUDAGraph()
    reset()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        reset()
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], eager_out[i]), (rep, i)
            for n, t in work[i].buffers().items():
                assert torch.equal(t, eager_state[i][n]), (rep, i, n)
        assert not work[0].tickets.any() and not work[1].tickets.any()
