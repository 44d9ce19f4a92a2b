"""fp64 CPU oracle for the attention forward pass.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It shares no code with
the HIP path.
"""
from .reference import (  # noqa: F401
    CAUSAL,
    CAUSAL_WINDOW,
    FULL,
    LOCAL_GLOBAL,
    MASK_KINDS,
    attention,
    effective_flops,
    global_set,
    kv_head,
    softmax_rows,
    visibility,
    visible_pair_count,
    weights,
)
from .decode import (  # noqa: F401
    DECODE_MASK_KINDS,
    decode_attention,
    decode_cache_bytes,
    decode_effective_flops,
    decode_visible_count,
    decode_visible_range,
)
from .cross import (  # noqa: F401
    CROSS_MASK_KINDS,
    cross_attention,
    cross_visible_pairs,
    cross_visible_range,
)
from .sparse import (  # noqa: F401
    bigbird_layout,
    block_sparse_attention,
    block_sparse_pairs,
    fixed_layout,
    strided_layout,
)
from .fp8 import (  # noqa: F401
    FP8_FORMATS,
    e4m3_decode,
    e5m2_decode,
    fp8_decode,
    fp8_attention,
    fp8_error_bound,
    fp8_tolerance,
)
