"""libw4a16: W4A16 linear layer (int4 weights, fp16/bf16 activations) for MI355X.

The computation lives in the hand-written HIP library ``libw4a16.so`` (C ABI
in ``include/w4a16.h``); this package is its Python binding.
"""
from ._binding import (  # noqa: F401
    ABI_VERSION, GEMV_MAX_M, LIB_PATH, PATH_AUTO, PATH_GEMM, PATH_GEMV, SIGNATURES,
    W4A16_BF16, W4A16_F16, W4A16Error,
    w4a16_abi_version, w4a16_check_args, w4a16_dequant, w4a16_last_error, w4a16_linear,
    w4a16_linear_path, w4a16_pack_weights, w4a16_pack_zeros, w4a16_select_path,
    w4a16_unpack_device, w4a16_unpack_weights, w4a16_unpack_zeros, w4a16_workspace_size,
    w4a16_linear_dense, w4a16_dense_workspace_size, w4a16_moe_linear, w4a16_reload_tuning, w4a16_plan,
    w4a16_linear_noalloc, NOALLOC_SCRATCH_BYTES,
)
