"""gfx950 (MI355X) W4A8 block-quantized matmul: Python binding of libq4.so.

The compute lives in hand-written HIP kernels behind the C ABI in
include/q4.h; this package only marshals torch device tensors to it.
"""
from ._lib import (  # noqa: F401
    EXPORTS, LIB_PATH, Q4Error, code_shape, debug_partials, debug_partials_fused, gemm, gemm_backward, gemm_packed, gemv, gemv_fused, lib, measure_empty,
    measure_stream_read, pack_weights,
    packed_bytes, q4k_gemm, q4k_gemm_work, q4k_gemm_backward, q4k_gemm_backward_noalloc, q4k_gemv, q4k_quantize_weights, quantize_act, quantize_weights,
    status_string,
)
