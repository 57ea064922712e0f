"""CPU oracle for KIVI-style quantized-KV decode attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import anything from this package.  The product path (the HIP library and its
Python binding) never imports, calls or links it, and this package imports
nothing from the product path.

It is a plain, slow, obviously correct numpy implementation of what the hot
path computes, written from the pages' definitions:

* ``quantizer``  -- the uniform asymmetric B-bit quantizer, keys grouped per
  channel over G tokens, values grouped per token over G channels, and the
  exact (fp64) dequantization.
* ``packing``    -- the documented uint32 tile layout of the codes.
* ``attention``  -- fp64 softmax attention of one query over a token set, the
  split (partial) form and its log-sum-exp merge.
* ``cache``      -- the streaming cache (prefill, append, flush, decode) in the
  library's documented buffer layouts, one (sequence, head) at a time.
* ``axis_ablation`` -- the four choices of grouping axis for keys and values
  and the key, score and output errors each gives (analysis, not parity).
* ``rope``       -- the rotary embedding applied to keys after dequantization
  (keys stored before the rotation) and the decode that uses it.
* ``sink``       -- the decode over an fp16 attention-sink segment followed by
  the cache's tokens.
* ``value_queue`` -- the cache whose values leave an fp16 queue of the newest
  R one token at a time (quantized per token as they leave), keys flushed R
  at a time; its prefill, append, key flush and decode.

Precision: the quantizer runs the fixed fp32 operation sequence stated in
``quantizer``; attention runs in fp64 on the exactly dequantized values.

Every function is pinned by CPU tests against facts the pages or mathematics
fix (hand-worked cases, brute force, closed forms, invariants); none is
"parity unpinned".
"""

from . import attention, axis_ablation, cache, packing, quantizer, rope, sink, value_queue  # noqa: F401
