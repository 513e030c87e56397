"""Python binding of libq4dec, the MI355X (gfx950) Q4_0 decode hot path.

Every function here only marshals arguments (torch tensors -> device pointers,
the current HIP stream) into the C ABI declared in include/q4dec.h; all
computation runs in the HIP kernels of libq4dec.so.  Importing fails loudly if
the library has not been built: there is no CPU fallback.
"""
from ._lib import (  # noqa: F401
    Q4Error,
    KVLayout,
    DecodeModel,
    argmax_rows,
    argmax_rows_ws,
    gqa_decode_attn,
    gqa_decode_attn_rope,
    gqa_decode_attn_workspace,
    lib,
    matvec_batched_workspace,
    IN_PLAIN,
    IN_RMSNORM,
    IN_SWIGLU,
    IN_GEGLU,
    OUT_PLAIN,
    OUT_SWIGLU,
    OUT_GEGLU,
    q4_0_matvec,
    q4_0_matvec_fused,
    q4_0_matvec_post_norm,
    q4_0_matvec_batched,
    q4_0_matvec_batched_noalloc,
    q8_0_matvec_batched,
    q8_0_matvec_fused,
    q8_0_gather,
    q8_0_matvec,
    qk_norm_rope,
    rmsnorm,
    rmsnorm_add,
    softcap,
    swiglu,
    geglu,
    version,
)
