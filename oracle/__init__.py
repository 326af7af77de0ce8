"""fp64 CPU oracle for sparse MLA forward. Test infrastructure only: imported by
the tests, the package smoke check and the benchmark's CPU-baseline leg, never by
the library."""

from .sparse_mla_oracle import (  # noqa: F401
    D_V,
    attend_row,
    bf16_bits_to_f64,
    decode_q,
    decode_rows,
    e4m3fn_table,
    lse_combine,
    softmax_weights,
    sparse_mla_fwd,
    sparse_mla_fwd_2seg,
    sparse_mla_fwd_2seg_torch,
    sparse_mla_fwd_torch,
)
from . import out_epilogue  # noqa: F401,E402  (inverse RoPE + MXFP8 output epilogue)
from . import indexer  # noqa: F401,E402  (fp8 MQA logits + top-k of the indexer)
