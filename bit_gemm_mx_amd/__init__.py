"""libmx: OCP Microscaling (MX) quantize / dequantize / block matmul on MI355X.

The compute runs in hand-written HIP kernels for gfx950 behind the C ABI of
``include/libmx.h`` (``libmx.so``); this package is its thin Python binding.
"""
from .binding import (  # noqa: F401
    BLOCK, MX_E2M1, MX_E4M3, LibMXError, MXTensor, block_matmul, block_matmul_f32b,
    block_matmul_quantize_a, dequantize, empty_mx, fold_scale, lib, quantize,
)
