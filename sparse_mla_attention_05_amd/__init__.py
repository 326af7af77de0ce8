"""Sparse multi-head latent attention (MLA) forward for MI355X (gfx950).

The compute path is libsparse_mla.so (hand-written HIP kernels behind a C ABI,
include/sparse_mla.h); this package holds its sources (csrc/), the in-tree
build script (build.py), a thin ctypes binding (_lib.py) and the seeded
synthetic input generators (inputs.py).
"""

from ._lib import (  # noqa: F401
    SparseMLAError,
    forward,
    forward2,
    load,
    sparse_mla_fwd,
    sparse_mla_fwd2,
    sparse_mla_fwd_epi,
    sparse_mla_fwd_ex,
    sparse_mla_indexer_logits,
    sparse_mla_indexer_topk,
    sparse_mla_is_supported,
    sparse_mla_out_epilogue,
    sparse_mla_plan,
    sparse_mla_plan2,
    sparse_mla_work_of,
)
