"""MI355X-native 4-bit block-quantized weight matmul (decode and A8 prefill)
and the decode-time read of a 4-bit K/V cache.

The compute lives in the HIP library ``libq4w.so`` (hand-written gfx950
kernels behind a C ABI declared in ``include/q4w.h``); this package is only
the argument-marshalling binding.  Import is lazy: ``synthetic`` works
without the library, while every compute call loads it and fails loudly if
it has not been built.
"""

from .binding import (  # noqa: F401
    Batch,
    Q4WError,
    a8_quantize_act,
    attn_decode,
    attn_decode_ws_bytes,
    a8w4_debug_block_acc,
    a8w4_gemm,
    a8w4_gemm_prepared,
    a8w4_prepare,
    a8w4_ws_bytes,
    batched_plan,
    batched_ws_bytes,
    gemv,
    gemv_noalloc,
    gemv_ws_bytes,
    lib,
    lib_path,
    pack,
    q4_gemv_skinny_raw,
    stream_read,
)
