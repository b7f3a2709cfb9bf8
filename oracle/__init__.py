"""CPU oracle for NVFP4 block quantization with ScaleSearch.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product
(``microscaling_fp4_block_amd``) never imports it.
"""
from .oracle import (  # noqa: F401
    F32,
    BF16,
    build,
    lib,
    e2m1_code,
    e4m3_encode,
    e4m3_value,
    block_sse,
    quantize,
    dequantize,
    quantize_kv_sink,
    dequantize_kv_sink,
    hadamard128,
    hadamard128_rht,
    quantize_rht,
    balance_exponent,
    balance_exponents,
    quantize_balanced,
    hadamard128_balanced,
    quantize_mxfp4,
    dequantize_mxfp4,
    mx_block_sse,
    attention_nvfp4,
    attention_kv_cache,
)
