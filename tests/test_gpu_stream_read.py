"""GPU check of the stream-read measurement aid (kivi_stream_read): every
16-byte piece of the buffer is read exactly once, whatever the grid, so the
XOR of all per-wave folds equals the XOR of every 32-bit word of the buffer
(computed on the host).  Sizes cover one piece, ragged tails of the unrolled
rounds, more workgroups than pieces and a buffer of the decode's size."""

import numpy as np
import pytest
import torch

from bit_kv_cache_decode_amd import kivi

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("pieces,workgroups", [
    (1, 1), (1, 7), (4097, 1), (4097, 3), (123457, 1024), (100, 256),
    (114491392 // 16, 1024), (114491392 // 16, 256),
])
def test_stream_read_folds_every_word_once(pieces, workgroups):
    rng = np.random.Generator(np.random.PCG64(77 + pieces))
    host = rng.integers(0, 2**32, size=pieces * 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((workgroups * 8,), -1, dtype=torch.int32, device="cuda")
    kivi.stream_read(src, workgroups, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(host)), (pieces, workgroups)
