"""ctypes binding of libgemm.so: the C entry points under the same names.

Argument marshalling only -- every step of C = A.B runs in the library's HIP kernels.
The library is loaded on first use; if it is not built (gemm_f32_amd/build.py) that use
raises LibraryNotBuilt: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import enum
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgemm.so")


class Order(enum.IntEnum):
    ROW_MAJOR = 0
    COL_MAJOR = 1


class Algo(enum.IntEnum):
    AUTO = 0
    NAIVE_UNCOALESCED = 1
    NAIVE = 2
    TILED = 3
    REGBLOCK = 4
    MFMA = 5
    MFMA_256x256 = 6
    MFMA_256x128 = 7
    MFMA_128x128 = 8
    MFMA_64x64 = 9
    SKINNY = 11
    MFMA_DMA = 12


class Status(enum.IntEnum):
    OK = 0
    ERR_INVALID_VALUE = 1
    ERR_UNSUPPORTED_DEVICE = 2
    ERR_LAUNCH = 3
    ERR_SCRATCH_TOO_SMALL = 4


class Fp8(enum.IntEnum):
    """gemm_fp8_t: the OCP 8-bit formats of gemm_fp8_f32acc's operands"""
    E4M3 = 0
    E5M2 = 1


class LibraryNotBuilt(ImportError):
    pass


class GemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = Status(status)
        lib = lib_handle()
        msg = lib.gemm_status_string(status).decode()
        if self.status == Status.ERR_LAUNCH:
            msg += f" (hipError_t {lib.gemm_last_hip_error()})"
        super().__init__(f"{what}: {msg}")


_lib = None


def lib_handle():
    """The loaded libgemm.so (loaded on first call)."""
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def _load():
    if not os.path.exists(_LIB_PATH):
        raise LibraryNotBuilt(
            f"{_LIB_PATH} is not built; build it with `python -m gemm_f32_amd.build` "
            "(hipcc, gfx950). There is no non-HIP fallback.")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    args = [i64, i64, i64, vp, i64, ci, vp, i64, ci, vp, i64, ci, vp]
    for name in ("gemm_f32", "gemm_bf16_f32acc"):
        f = getattr(lib, name)
        f.argtypes, f.restype = args, ci
    for name in ("gemm_f32_algo", "gemm_bf16_f32acc_algo"):
        f = getattr(lib, name)
        f.argtypes, f.restype = [ci] + args, ci
    lib.gemm_status_string.argtypes, lib.gemm_status_string.restype = [ci], ctypes.c_char_p
    lib.gemm_last_hip_error.argtypes, lib.gemm_last_hip_error.restype = [], ci
    lib.gemm_last_kernel.argtypes, lib.gemm_last_kernel.restype = [], ctypes.c_char_p
    lib.gemm_version.argtypes, lib.gemm_version.restype = [], ctypes.c_char_p
    lib.gemm_plan.argtypes = [ci, i64, i64, i64, ci, ci, ci, ci, ctypes.POINTER(ctypes.c_char_p),
                              ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_size_t)]
    lib.gemm_plan.restype = ci
    lib.gemm_workspace_size.argtypes = [ci, i64, i64, i64, ci, ci, ci]
    lib.gemm_workspace_size.restype = ctypes.c_size_t
    for name in ("gemm_f32_ws", "gemm_bf16_f32acc_ws", "gemm_f16_f32acc_ws"):
        f = getattr(lib, name)
        f.argtypes, f.restype = args[:-1] + [vp, ctypes.c_size_t, vp], ci
    lib.gemm_f16_f32acc.argtypes, lib.gemm_f16_f32acc.restype = args, ci
    lib.gemm_f16_f32acc_algo.argtypes, lib.gemm_f16_f32acc_algo.restype = [ci] + args, ci
    batched = [i64, i64, i64, i64, vp, i64, i64, ci, vp, i64, i64, ci, vp, i64, i64, ci, vp]
    for name in ("gemm_f32_strided_batched", "gemm_bf16_f32acc_strided_batched",
                 "gemm_f16_f32acc_strided_batched"):
        f = getattr(lib, name)
        f.argtypes, f.restype = batched, ci
    for name in ("gemm_bf16_f32acc_fused", "gemm_f16_f32acc_fused", "gemm_f32_fused"):
        f = getattr(lib, name)
        f.argtypes, f.restype = args[:-1] + [ctypes.POINTER(EpilogueStruct), vp], ci
    lib.gemm_bf16_f32acc_noalloc.argtypes, lib.gemm_bf16_f32acc_noalloc.restype = args, ci
    lib.gemm_fp8_f32acc.argtypes = [i64, i64, i64, vp, i64, ci, ci, vp, i64, ci, ci, vp, i64, ci, vp]
    lib.gemm_fp8_f32acc.restype = ci
    return lib


class Act(enum.IntEnum):
    """gemm_activation_t"""
    NONE = 0
    RELU = 1
    GELU = 2


class Out(enum.IntEnum):
    """gemm_out_t"""
    F32 = 0
    BF16 = 1


class EpilogueStruct(ctypes.Structure):
    """gemm_epilogue_t"""
    _fields_ = [("alpha", ctypes.c_float), ("beta", ctypes.c_float), ("bias", ctypes.c_void_p),
                ("activation", ctypes.c_int), ("out_type", ctypes.c_int)]


EXPORTED = ("gemm_f32", "gemm_bf16_f32acc", "gemm_f32_algo", "gemm_bf16_f32acc_algo",
            "gemm_status_string", "gemm_last_hip_error", "gemm_last_kernel", "gemm_version",
            "gemm_plan", "gemm_workspace_size", "gemm_f32_ws", "gemm_bf16_f32acc_ws",
            "gemm_f16_f32acc", "gemm_f16_f32acc_algo", "gemm_f16_f32acc_ws",
            "gemm_f32_strided_batched", "gemm_bf16_f32acc_strided_batched",
            "gemm_f16_f32acc_strided_batched", "gemm_bf16_f32acc_fused", "gemm_f16_f32acc_fused",
            "gemm_bf16_f32acc_noalloc", "gemm_fp8_f32acc", "gemm_f32_fused")

# bytes of the static scratch behind gemm_bf16_f32acc_noalloc (GEMM_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20

# dtype codes of gemm_plan / gemm_workspace_size (every 8-bit format pairing is code 3)
DTYPE_CODE = {"f32": 0, "bf16": 1, "f16": 2, "fp8": 3, "e4m3": 3, "e5m2": 3, "e4m3_e5m2": 3, "e5m2_e4m3": 3}


def library_path() -> str:
    return _LIB_PATH


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise GemmError(rc, what)


def gemm_f32(M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, stream=0):
    """C = A.B, FP32.  A, B, C are device pointers (ints); stream a hipStream_t (int)."""
    _check(lib_handle().gemm_f32(M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, stream),
           "gemm_f32")


def gemm_bf16_f32acc(M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, stream=0):
    """C = A.B with bf16 A and B (bit patterns), FP32 accumulate and FP32 C."""
    _check(lib_handle().gemm_bf16_f32acc(M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c,
                                 stream), "gemm_bf16_f32acc")


def gemm_f32_algo(algo, M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, stream=0):
    _check(lib_handle().gemm_f32_algo(int(algo), M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc,
                              order_c, stream), "gemm_f32_algo")


def gemm_bf16_f32acc_algo(algo, M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c,
                          stream=0):
    _check(lib_handle().gemm_bf16_f32acc_algo(int(algo), M, N, K, A, lda, order_a, B, ldb, order_b, C,
                                      ldc, order_c, stream), "gemm_bf16_f32acc_algo")


def gemm_status_string(status: int) -> str:
    return lib_handle().gemm_status_string(int(status)).decode()


def gemm_last_hip_error() -> int:
    return lib_handle().gemm_last_hip_error()


def gemm_last_kernel() -> str:
    return lib_handle().gemm_last_kernel().decode()


def gemm_version() -> str:
    return lib_handle().gemm_version().decode()


def gemm_plan(dtype, M, N, K, order_a, order_b, order_c, cus=256, with_workspace=False):
    """(kernel, core_rows, core_cols) the default choice would run, plus the split-K workspace
    bytes when with_workspace; no device needed."""
    kernel, rows, cols, ws = ctypes.c_char_p(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t()
    _check(lib_handle().gemm_plan(DTYPE_CODE[dtype], M, N, K, order_a, order_b, order_c, cus,
                                  ctypes.byref(kernel), ctypes.byref(rows), ctypes.byref(cols),
                                  ctypes.byref(ws)), "gemm_plan")
    out = (kernel.value.decode(), rows.value, cols.value)
    return out + (ws.value,) if with_workspace else out


def gemm_workspace_size(dtype, M, N, K, order_a, order_b, order_c) -> int:
    """Workspace bytes with which the _ws calls split K on the current device (0: no split)."""
    return lib_handle().gemm_workspace_size(DTYPE_CODE[dtype], M, N, K, order_a, order_b, order_c)


def gemm_f32_ws(M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, workspace, workspace_bytes,
                stream=0):
    """gemm_f32 with a caller's workspace (device pointer, bytes) for split-K."""
    _check(lib_handle().gemm_f32_ws(M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, workspace,
                                    workspace_bytes, stream), "gemm_f32_ws")


def gemm_f16_f32acc(M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, stream=0):
    """C = A.B with IEEE fp16 A and B (bit patterns), FP32 accumulate and FP32 C."""
    _check(lib_handle().gemm_f16_f32acc(M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, stream),
           "gemm_f16_f32acc")


def gemm_f16_f32acc_algo(algo, M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, stream=0):
    _check(lib_handle().gemm_f16_f32acc_algo(int(algo), M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc,
                                             order_c, stream), "gemm_f16_f32acc_algo")


def gemm_f16_f32acc_ws(M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, workspace,
                       workspace_bytes, stream=0):
    """gemm_f16_f32acc with a caller's workspace (device pointer, bytes) for split-K."""
    _check(lib_handle().gemm_f16_f32acc_ws(M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c,
                                           workspace, workspace_bytes, stream), "gemm_f16_f32acc_ws")


def gemm_bf16_f32acc_ws(M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, workspace,
                        workspace_bytes, stream=0):
    """gemm_bf16_f32acc with a caller's workspace (device pointer, bytes) for split-K."""
    _check(lib_handle().gemm_bf16_f32acc_ws(M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c,
                                            workspace, workspace_bytes, stream), "gemm_bf16_f32acc_ws")


def gemm_bf16_f32acc_noalloc(M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, stream=0):
    """gemm_bf16_f32acc_ws with the library's static scratch as workspace: allocates nothing."""
    _check(lib_handle().gemm_bf16_f32acc_noalloc(M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c,
                                                 stream), "gemm_bf16_f32acc_noalloc")


def gemm_fp8_f32acc(M, N, K, A, lda, order_a, format_a, B, ldb, order_b, format_b, C, ldc, order_c, stream=0):
    """C = A.B with 8-bit A and B (bit patterns; format_* an Fp8), FP32 accumulate and FP32 C.
    A row-major, B column-major."""
    _check(lib_handle().gemm_fp8_f32acc(M, N, K, A, lda, order_a, int(format_a), B, ldb, order_b, int(format_b),
                                        C, ldc, order_c, stream), "gemm_fp8_f32acc")


# --- torch tensors -> (pointer, leading dimension, order) ------------------------------
def gemm_f32_strided_batched(batch, M, N, K, A, lda, stride_a, order_a, B, ldb, stride_b, order_b,
                             C, ldc, stride_c, order_c, stream=0):
    """C_z = A_z.B_z for z < batch, FP32; entry z at A + z*stride_a etc. (element strides)."""
    _check(lib_handle().gemm_f32_strided_batched(batch, M, N, K, A, lda, stride_a, order_a, B, ldb, stride_b,
                                                 order_b, C, ldc, stride_c, order_c, stream),
           "gemm_f32_strided_batched")


def gemm_bf16_f32acc_strided_batched(batch, M, N, K, A, lda, stride_a, order_a, B, ldb, stride_b, order_b,
                                     C, ldc, stride_c, order_c, stream=0):
    """Strided batch of bf16 products (bit patterns), FP32 accumulate and FP32 C."""
    _check(lib_handle().gemm_bf16_f32acc_strided_batched(batch, M, N, K, A, lda, stride_a, order_a, B, ldb,
                                                         stride_b, order_b, C, ldc, stride_c, order_c, stream),
           "gemm_bf16_f32acc_strided_batched")


def gemm_f16_f32acc_strided_batched(batch, M, N, K, A, lda, stride_a, order_a, B, ldb, stride_b, order_b,
                                    C, ldc, stride_c, order_c, stream=0):
    """Strided batch of IEEE fp16 products (bit patterns), FP32 accumulate and FP32 C."""
    _check(lib_handle().gemm_f16_f32acc_strided_batched(batch, M, N, K, A, lda, stride_a, order_a, B, ldb,
                                                        stride_b, order_b, C, ldc, stride_c, order_c, stream),
           "gemm_f16_f32acc_strided_batched")


def _fused(name, M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, alpha, beta, bias, activation,
           out_type, stream):
    epi = EpilogueStruct(alpha, beta, bias or None, int(activation), int(out_type))
    _check(getattr(lib_handle(), name)(M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c,
                                       ctypes.byref(epi), stream), name)


def gemm_bf16_f32acc_fused(M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, alpha=1.0, beta=0.0,
                           bias=0, activation=Act.NONE, out_type=Out.F32, stream=0):
    """C = act(alpha*A.B + beta*C + bias) with bf16 inputs; C float or bf16 bits per out_type;
    bias a device pointer to N floats (0: none)."""
    _fused("gemm_bf16_f32acc_fused", M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, alpha, beta,
           bias, activation, out_type, stream)


def gemm_f16_f32acc_fused(M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, alpha=1.0, beta=0.0,
                          bias=0, activation=Act.NONE, out_type=Out.F32, stream=0):
    """gemm_bf16_f32acc_fused for IEEE fp16 inputs."""
    _fused("gemm_f16_f32acc_fused", M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, alpha, beta,
           bias, activation, out_type, stream)


def gemm_f32_fused(M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, alpha=1.0, beta=0.0,
                   bias=0, activation=Act.NONE, out_type=Out.F32, stream=0):
    """gemm_bf16_f32acc_fused for FP32 inputs (row-major A, column-major B, K >= 32)."""
    _fused("gemm_f32_fused", M, N, K, A, lda, order_a, B, ldb, order_b, C, ldc, order_c, alpha, beta,
           bias, activation, out_type, stream)


def operand_layout(t) -> tuple[int, int]:
    """(ld, order) of a 2-D tensor whose memory is row- or column-major with padding."""
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    R, C = t.shape
    s0, s1 = t.stride()
    if s1 == 1 and s0 >= max(1, C):
        return s0, Order.ROW_MAJOR
    if s0 == 1 and s1 >= max(1, R):
        return s1, Order.COL_MAJOR
    if R <= 1 and s1 == 1:
        return max(1, C), Order.ROW_MAJOR
    if C <= 1 and s0 == 1:
        return max(1, R), Order.COL_MAJOR
    raise ValueError(f"strides {t.stride()} are neither row- nor column-major")


def matmul(a, b, out=None, algo: Algo = Algo.AUTO, stream=None):
    """out = a @ b for torch device tensors, through libgemm on the current stream.

    a: (M, K), b: (K, N), both float32 (FP32 path), both bfloat16 or both float16 (16-bit
    inputs, FP32 accumulate).  out: float32 (M, N), row- or column-major; allocated row-major
    if None.
    """
    import torch
    if a.dtype != b.dtype or a.dtype not in (torch.float32, torch.bfloat16, torch.float16):
        raise TypeError("a and b must both be float32, both bfloat16 or both float16")
    M, K = a.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {a.shape} x {b.shape}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (M, N):
        raise ValueError("out must be float32 of shape (M, N)")
    lda, oa = operand_layout(a)
    ldb, ob = operand_layout(b)
    ldc, oc = operand_layout(out)
    s = torch.cuda.current_stream(a.device).cuda_stream if stream is None else stream
    args = (M, N, K, a.data_ptr(), lda, oa, b.data_ptr(), ldb, ob, out.data_ptr(), ldc, oc, s)
    if a.dtype == torch.float32:
        gemm_f32_algo(algo, *args)
    elif a.dtype == torch.bfloat16:
        gemm_bf16_f32acc_algo(algo, *args)
    else:
        gemm_f16_f32acc_algo(algo, *args)
    return out
