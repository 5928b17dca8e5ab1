"""Test-only oracle for the W4A16 weight-only GEMM/GEMV (see w4a16_oracle).

This package is test infrastructure. Only the tests, the smoke entry point and the
benchmark's CPU-baseline leg may import it; the product path never does.
"""
from .w4a16_oracle import (  # noqa: F401
    GROUP_SIZE, NIBBLE_K, quantize, pack, unpack, dequant, dequant_fp16, matmul, quantize_pack,
)
from .w4a8_oracle import (  # noqa: F401
    E4M3_MAX, e4m3_decode, e4m3_encode, quantize_activations, activation_block_sums, weight_values, matmul_w4a8,
)
