"""kivi_decode_attn_noalloc (the decode with the library's own device array as
scratch, for callers that cannot allocate) against kivi_decode_attn, through
the C ABI: the same kernels, so the outputs must be identical bit for bit.
Two calls in a row share the array, the second on a smaller input; sizes
past the array's limits are refused before anything is launched."""

import numpy as np
import pytest
import torch

from bit_kv_cache_decode_amd import kivi
from tests.gpu_common import gpu_cache, workload

pytestmark = pytest.mark.gpu


def _both(c, w):
    q = torch.from_numpy(w.q).cuda()
    d = c.dims
    out = torch.full((d.batch, d.heads, d.head_dim), float("nan"), dtype=torch.float32,
                     device="cuda")
    kivi.decode_attn_noalloc(c, q, w.config.sm_scale, out)
    ref = kivi.decode_attn(c, q, w.config.sm_scale)
    torch.cuda.synchronize()
    assert c.status_bits() == 0
    return out.cpu(), ref.cpu()


def test_noalloc_matches_decode_attn_on_two_calls_in_a_row():
    # first call: 2 x 32 heads, each split over several workgroups (the
    # capacity sets the split), so the array holds partials and counters
    w = workload(2, batch=2)
    big = gpu_cache(w, capacity=65536)
    assert kivi.decode_splits(big.dims) > 1
    out, ref = _both(big, w)
    assert torch.equal(out, ref)
    # second call: a smaller input (one sequence, a shorter capacity; the
    # split plan again fills the chip, with 8 splits per head) on the same
    # array, which still holds the first call's partials in other places
    w1 = workload(2, batch=1)
    small = gpu_cache(w1, capacity=8192)
    assert kivi.decode_splits(small.dims) > 1 and small.dims.batch < big.dims.batch
    assert small.nbytes() < big.nbytes()
    out, ref = _both(small, w1)
    assert torch.equal(out, ref)
    # and the single-workgroup plan (no partials at all)
    tiny = workload(1)
    c = gpu_cache(tiny)
    out, ref = _both(c, tiny)
    assert torch.equal(out, ref)


def test_noalloc_refuses_sizes_past_the_array():
    c = kivi.KiviCache(128, 64, 128, 2, 32, 32, 32)      # 8192 (sequence, head) pairs
    q = torch.zeros((128, 64, 128), dtype=torch.float16, device="cuda")
    out = torch.zeros((128, 64, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(kivi.KiviError) as e:
        kivi.decode_attn_noalloc(c, q, 1.0, out)
    assert e.value.code == kivi.KIVI_ENOSPC
    torch.cuda.synchronize()
    assert not out.any()
