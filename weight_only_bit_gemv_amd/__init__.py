"""MI355X (gfx950) W4A16 weight-only GEMM/GEMV: y = x . dequant(Wq), and its W4A8 variant.

The compute lives in libw4a16.so (hand-written HIP kernels behind a C ABI, include/w4a16.h);
this package only marshals arguments to it. Importing the package loads the library and
raises if it cannot, so there is no silent fallback path.
"""
from ._binding import (  # noqa: F401
    GROUP_SIZE, LIB_PATH, W4A16Error, hip_runtimes_loaded, w4a16_pack, w4a16_unpack, w4a16_plan, w4a16_matmul,
    w4a16_matmul_ex, w4a16_matmul_noalloc, w4a16_matmul_grouped, w4a16_autotune, w4a16_set_plan,
    w4a16_clear_plans, w4a16_dequant, w4a16_version, strerror, load, w4a8_quantize, w4a8_matmul, w4a8_sum_stride,
    W4A16_OK, W4A16_ERR_INVALID_ARG, W4A16_ERR_UNSUPPORTED, W4A16_ERR_ALIGNMENT,
    W4A16_ERR_NONFINITE, W4A16_ERR_HIP, W4A16_KERNEL_AUTO, W4A16_KERNEL_SKINNY,
    W4A16_KERNEL_PREFILL, W4A16_TILE_LDS, W4A16_TILE_REGISTER_B, W4A16_TILE_ASYNC,
    W4A16_LAYOUT_LINEAR, W4A16_LAYOUT_INTERLEAVED,
)

load()
