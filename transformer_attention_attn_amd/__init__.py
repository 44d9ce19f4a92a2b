"""MI355X-native fused attention forward: masked, grouped-query
scaled dot-product attention in hand-written gfx950 HIP kernels.

The library is libattn.so (C ABI in include/attn.h); this package is a thin
ctypes binding over it.  Build it with
``python -m transformer_attention_attn_amd.build``.
"""
from ._binding import (  # noqa: F401
    DTYPE_BF16,
    DTYPE_FP32,
    DTYPE_FP8,
    DTYPE_FP8_E5M2,
    EXPORTS,
    LIB_PATH,
    MASK_CAUSAL,
    MASK_CAUSAL_WINDOW,
    MASK_FULL,
    MASK_LOCAL_GLOBAL,
    MASKS,
    MAX_GLOBAL,
    SPARSE_BLOCK,
    SPARSE_MAX_BLOCKS,
    STATUS,
    AttnError,
    FwdArgs,
    check_devices,
    decode,
    decode_noalloc,
    decode_noalloc_raw,
    decode_raw,
    decode_workspace_bytes,
    decode_workspace_status,
    fwd,
    fwd_ex,
    fwd_ex_raw,
    fwd_raw,
    layout_bigbird,
    layout_fixed,
    layout_strided,
    layout_words,
    load,
    plan,
    plan_status,
    status_string,
    version,
)
