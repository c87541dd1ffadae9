"""Block-sparse (BSR / paged) attention for AMD Instinct MI355X (gfx950).

The compute path lives in the HIP library ``libbsr_attn.so`` (C ABI:
``include/bsr_attn.h``); ``block_sparse_paged_bsr_amd.api`` is its Python binding.
Importing this package does not load the library; the first binding call does, and
raises if the library has not been built.  The seeded synthetic workloads used by the
tests and the benchmark live outside the package, in ``workloads.py`` at the repository
root.
"""

__all__ = ["api", "build"]
