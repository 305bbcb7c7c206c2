"""Single-query GQA decode attention on MI355X: Python binding of libgqa_decode.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels of the C library (``include/gqa_decode.h``).  PyTorch supplies device
memory and the stream.  There is no fallback: if the library has not been
built, importing this package raises.
"""
from ._binding import (  # noqa: F401
    GQA_BF16,
    GQA_KV_CONTIGUOUS,
    GQA_KV_PAGED,
    GQA_KV_PAGED_XSPLIT,
    DecodeArgs,
    GQA_F16,
    GQA_POLICY_FUSED_MERGE,
    GQA_POLICY_VALU_DOT2,
    GqaError,
    Policy,
    decode,
    decode_contiguous,
    decode_noalloc,
    NOALLOC_SCRATCH_BYTES,
    decode_xsplit,
    X,
    lib,
    library_path,
    policy_default,
    policy_pages,
    status_string,
    check_block_table,
    workspace_size,
    EXPORTED_SYMBOLS,
    PreparedCall,
    prepare,
)
