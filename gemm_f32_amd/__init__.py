"""libgemm for MI355X: dense C = A.B with hand-written HIP kernels for gfx950.

The entry points mirror include/gemm.h.  libgemm.so (built in-tree by
gemm_f32_amd/build.py) is loaded on first use and its absence is an error: there is no
fallback path.
"""
from .binding import (  # noqa: F401
    EXPORTED, Algo, GemmError, Order, Status, gemm_bf16_f32acc, gemm_bf16_f32acc_algo,
    gemm_f32, gemm_f32_algo, gemm_last_hip_error, gemm_last_kernel, gemm_status_string,
    gemm_version, gemm_plan, gemm_workspace_size, gemm_f32_ws, gemm_bf16_f32acc_ws,
    gemm_f16_f32acc, gemm_f16_f32acc_algo, gemm_f16_f32acc_ws,
    gemm_f32_strided_batched, gemm_bf16_f32acc_strided_batched, gemm_f16_f32acc_strided_batched,
    gemm_bf16_f32acc_fused, gemm_f16_f32acc_fused, gemm_bf16_f32acc_noalloc, NOALLOC_SCRATCH_BYTES,
    gemm_fp8_f32acc, Fp8, gemm_f32_fused, Act, Out, lib_handle, library_path, LibraryNotBuilt, matmul, operand_layout,
)
