"""One GPU's share of Ulysses sequence parallelism on MI355X (gfx950).

The hot path -- sequence->head pack, causal GQA/varlen attention forward and
backward for one head group, head->sequence unpack -- runs in hand-written HIP
kernels behind the C ABI declared in include/ulysses.h. This package is the
thin Python binding of that library (same names, argument marshalling only)
plus its build step.
"""
from ._lib import (  # noqa: F401
    LIB_NAME,
    SIGNATURES,
    ULY_BF16,
    ULY_ERR_HIP,
    ULY_ERR_INVALID_ARG,
    ULY_ERR_UNSUPPORTED,
    ULY_F32,
    ULY_MAX_P,
    ULY_NOALLOC_SCRATCH_BYTES,
    ULY_OK,
    UlyssesError,
    attn_bwd,
    attn_bwd_ex,
    attn_bwd_accumulate,
    attn_bwd_noalloc,
    attn_bwd_workspace_size,
    attn_fwd,
    attn_fwd_from_shards,
    attn_merge,
    last_error,
    lib,
    lib_path,
    uly_check_cu_seqlens,
    ulysses_pack,
    ulysses_pack_heads,
    ulysses_pack_multi,
    ulysses_pack_qkv,
    ulysses_unpack,
    ulysses_unpack_heads,
    ulysses_unpack_multi,
    ulysses_unpack_qkv,
)
