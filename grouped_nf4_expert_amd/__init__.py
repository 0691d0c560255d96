"""grouped_nf4_expert_amd -- grouped NF4 expert GEMM (W4A16) for MI355X (gfx950).

The compute lives in ``libgnf4.so`` (hand-written HIP, C ABI declared in
``include/gnf4.h``).  ``grouped_nf4_expert_amd.gnf4`` is the thin Python
binding over it: argument marshalling only, every step runs in the library's
kernels.  Importing this package loads nothing; the library is opened on the
first call and a missing library is an error, never a fallback.
"""

__all__ = ["gnf4", "workloads"]
