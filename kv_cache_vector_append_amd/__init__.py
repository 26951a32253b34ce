"""TurboQuant-style compressed KV cache for AMD Instinct MI355X (gfx950).

The work happens in the HIP library ``libtq_hip.so`` behind the C ABI of
``include/tq.h``; this package only marshals torch tensors into those calls.
"""
from ._lib import (  # noqa: F401
    CacheBuffers,
    Config,
    TQ_MAX_CONTEXT,
    TQ_STATIC_WORKSPACE_BYTES,
    TQ_STATUS_BAD_PAGE,
    TQ_STATUS_BAD_SLOT,
    TQ_STATUS_CAPACITY,
    TQError,
    allocate_cache,
    build_id,
    decode_attention,
    decode_attention_static,
    decode_workspace_bytes,
    dequantize,
    exported_symbols,
    init_codebooks,
    key_block_bytes,
    load_library,
    params_bytes,
    quantize_append,
    value_block_bytes,
)
