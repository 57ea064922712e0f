"""KIVI-style quantized-KV decode attention for MI355X (gfx950).

The compute path is the HIP library ``libkivi.so`` built from ``csrc/``; the
Python layer (``kivi``) only marshals device pointers and streams through its
C ABI.  ``workloads`` draws seeded synthetic inputs and counts bytes.

Importing this package does not load the library; ``kivi.lib()`` does, and
raises if the shared object is missing.
"""

__all__ = ["kivi", "workloads"]
