"""MI355X (gfx950) hybrid SWA/global attention of the MiMo-V2-Flash decoder.

The compute lives in ``libmimo_attn.so`` (hand-written HIP, C ABI in ``include/mimo_attn.h``);
this package is its thin Python binding plus the per-layer dispatch from
``hybrid_layer_pattern``.
"""
from .binding import (  # noqa: F401
    BF16,
    CACHE_FP8_E4M3,
    CACHE_SAME,
    EXPORTS,
    F32,
    LAYER_GLOBAL,
    LAYER_SWA,
    MIMO_ERR_HIP,
    MIMO_ERR_INVALID_ARG,
    MIMO_ERR_UNSUPPORTED,
    MIMO_ERR_WORKSPACE,
    MIMO_OK,
    MimoAttnError,
    Params,
    RouterParams,
    check_params,
    decode,
    decode_workspace_size,
    decode_noalloc,
    decode_noalloc_max_bytes,
    extend,
    extend_workspace_size,
    last_error,
    layer_prefill,
    layer_workspace_size,
    lib,
    prefill,
    prefill_workspace_size,
    router_check_params,
    router_topk,
)
from .layers import (  # noqa: F401
    HybridAttentionConfig,
    LayerSpec,
    layer_spec,
    layer_specs,
    rope_dims_from_factor,
)
