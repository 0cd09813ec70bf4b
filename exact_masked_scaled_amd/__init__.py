"""Exact masked scaled dot-product attention for MI355X (gfx950).

The compute path is the C-ABI library ``libattn_mi355x.so`` (hand-written HIP
kernels); ``attn`` is its thin ctypes binding.  Importing this package does not
load the library; the first call does, and raises if it is missing.
"""

__all__ = ["workloads"]
