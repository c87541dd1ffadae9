"""Block-sparse (BSR / paged) attention for AMD Instinct MI355X (gfx950).

The compute path lives in the HIP library ``libbsr_attn.so`` (C ABI:
``include/bsr_attn.h``); ``block_sparse_paged_bsr_amd.api`` is its Python binding and
``block_sparse_paged_bsr_amd.inputs`` builds seeded synthetic workloads.  Importing
this package does not load the library; the first binding call does, and raises if
the library has not been built.
"""

__all__ = ["api", "inputs", "build"]
