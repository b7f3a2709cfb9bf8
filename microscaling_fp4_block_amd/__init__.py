"""NVFP4 block quantization with ScaleSearch on MI355X (gfx950).

The compute path is the HIP library ``libnvfp4.so`` (C ABI in
``include/nvfp4.h``); this package is its thin Python binding.
"""
from .nvfp4 import (  # noqa: F401
    LIB_PATH,
    NVFP4Error,
    attention,
    attention_kv_cache,
    attention_split_workspace_bytes,
    balance_exponents,
    dequantize,
    dequantize_kv_sink,
    global_scale,
    hadamard128,
    hw_self_check,
    kv_append,
    kv_append_dev,
    kv_append2_dev,
    kv_cache_alloc,
    kv_length,
    load,
    mxfp4_dequantize,
    mxfp4_quantize,
    quantize,
    quantize_kv_sink,
    quantize_noalloc,
    workspace_bytes,
)
