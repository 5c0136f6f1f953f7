"""Tree-verification hot path of Medusa/EAGLE-style speculative decoding on MI355X (gfx950).

The compute lives in ``libspectree.so`` (hand-written HIP kernels behind a C ABI declared
in ``include/spectree.h``).  :mod:`.binding` is a thin ctypes layer over it that marshals
torch device tensors and the current HIP stream; :mod:`.workloads` draws seeded synthetic
inputs.  Importing this package loads nothing; the library is loaded on first use and a
missing library is an error, never a fallback.
"""

__all__ = ["binding", "workloads"]
