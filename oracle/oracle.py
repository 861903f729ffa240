"""ctypes front end of the C oracle (oracle.c) -- TEST INFRASTRUCTURE ONLY.

The oracle computes C[i][j] = sum_k A[i][k] * B[k][j] in double, k ascending, on the
exact fp32, bf16, fp16 or 8-bit (OCP E4M3 / E5M2) input values, and D[i][j] = sum_k
|A[i][k] * B[k][j]|, the scale the parity tolerance is normalised by.  See oracle.c for the
cited definition.  8-bit operands are uint8 bit patterns whose format is named by the fmt_a /
fmt_b arguments ("e4m3" or "e5m2").
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

F32 = 0
BF16 = 1
F16 = 2
E4M3 = 3
E5M2 = 4
FP8_CODES = {"e4m3": E4M3, "e5m2": E5M2}


def library_path() -> str:
    return _LIB


def build(src: str = _SRC, out: str = _LIB, extra_flags: tuple = ()) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Werror",
           *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(path: str | None = None):
    """Load (building first if absent) the oracle library; returns the ctypes handle."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)
    lib.oracle_gemm.argtypes = [i64, i64, i64, ctypes.c_int, vp, i64, ctypes.c_int,
                                vp, i64, ctypes.c_int, dp, dp, ctypes.POINTER(i64)]
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_gemm_sampled.argtypes = [i64, i64, i64, ctypes.c_int, vp, i64, ctypes.c_int,
                                        vp, i64, ctypes.c_int, ctypes.POINTER(i64),
                                        ctypes.POINTER(i64), i64, dp, dp]
    lib.oracle_gemm_sampled.restype = ctypes.c_int
    lib.oracle_gemm_ab.argtypes = [i64, i64, i64, ctypes.c_int, vp, i64, ctypes.c_int,
                                   ctypes.c_int, vp, i64, ctypes.c_int, dp, dp, ctypes.POINTER(i64)]
    lib.oracle_gemm_ab.restype = ctypes.c_int
    lib.oracle_gemm_sampled_ab.argtypes = [i64, i64, i64, ctypes.c_int, vp, i64, ctypes.c_int,
                                           ctypes.c_int, vp, i64, ctypes.c_int, ctypes.POINTER(i64),
                                           ctypes.POINTER(i64), i64, dp, dp]
    lib.oracle_gemm_sampled_ab.restype = ctypes.c_int
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def _dtype_code(buf: np.ndarray, fmt=None) -> int:
    if buf.dtype == np.uint8:
        if fmt not in FP8_CODES:
            raise TypeError("8-bit operands need their format: fmt 'e4m3' or 'e5m2'")
        return FP8_CODES[fmt]
    if buf.dtype == np.float32:
        return F32
    if buf.dtype == np.uint16:
        return BF16
    if buf.dtype == np.float16:
        return F16
    raise TypeError(f"oracle operands are fp32, bf16 bits (uint16), fp16 or fp8 bits (uint8), got {buf.dtype}")


def gemm(M, N, K, A, lda, order_a, B, ldb, order_b, lib=None, return_macs=False, fmt_a=None, fmt_b=None):
    """Full product: returns (C, D) as M x N float64 arrays (and the MAC count if asked)."""
    lib = lib or load()
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    da, db = _dtype_code(A, fmt_a), _dtype_code(B, fmt_b)
    if da in (F32, BF16, F16) or db in (F32, BF16, F16):
        assert da == db, "operands of different types are 8-bit formats only"
    C = np.zeros((M, N), dtype=np.float64)
    D = np.zeros((M, N), dtype=np.float64)
    macs = ctypes.c_int64(-1)
    dp = ctypes.POINTER(ctypes.c_double)
    rc = lib.oracle_gemm_ab(M, N, K, da, A.ctypes.data, lda, order_a, db, B.ctypes.data, ldb, order_b,
                            C.ctypes.data_as(dp), D.ctypes.data_as(dp), ctypes.byref(macs))
    if rc != 0:
        raise ValueError("oracle_gemm rejected its arguments")
    return (C, D, macs.value) if return_macs else (C, D)


def gemm_sampled(M, N, K, A, lda, order_a, B, ldb, order_b, rows, cols, lib=None, fmt_a=None, fmt_b=None):
    """C and D at the (rows[t], cols[t]) elements only."""
    lib = lib or load()
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    da, db = _dtype_code(A, fmt_a), _dtype_code(B, fmt_b)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    C = np.zeros(rows.size, dtype=np.float64)
    D = np.zeros(rows.size, dtype=np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int64)
    rc = lib.oracle_gemm_sampled_ab(M, N, K, da, A.ctypes.data, lda, order_a, db, B.ctypes.data, ldb,
                                    order_b, rows.ctypes.data_as(ip), cols.ctypes.data_as(ip),
                                    rows.size, C.ctypes.data_as(dp), D.ctypes.data_as(dp))
    if rc != 0:
        raise ValueError("oracle_gemm_sampled rejected its arguments")
    return C, D


def gemm_strided_batched(batch, M, N, K, A, lda, stride_a, order_a, B, ldb, stride_b, order_b, lib=None):
    """A strided batch, entry by entry: (C, D) as batch x M x N float64 arrays.

    Entry z is the full product (gemm above) of the M x K matrix whose element (0, 0) sits at
    position z*stride_a of the flat buffer A and the K x N matrix at z*stride_b of B, each
    with its own leading dimension and order.  This is what a strided batched GEMM means:
    one independent product per entry ("A06 - Tiled Matrix Multiply (GEMM)", section "2.
    First Principles", the per-head attention products).
    """
    A = np.ascontiguousarray(A).reshape(-1)
    B = np.ascontiguousarray(B).reshape(-1)
    C = np.zeros((batch, M, N), dtype=np.float64)
    D = np.zeros((batch, M, N), dtype=np.float64)
    for z in range(batch):
        a = A[z * stride_a:]
        b = B[z * stride_b:]
        if M and N and K:
            assert a.size >= _extent(M, K, lda, order_a) and b.size >= _extent(K, N, ldb, order_b), \
                "a batch entry runs past the end of its buffer"
        C[z], D[z] = gemm(M, N, K, a, lda, order_a, b, ldb, order_b, lib=lib)
    return C, D


ACT_NONE, ACT_RELU, ACT_GELU = 0, 1, 2


def epilogue(C, D, alpha=1.0, beta=0.0, C_old=None, bias=None, activation=ACT_NONE):
    """Fused epilogue on the exact product, in float64: (Y, S) with

        Y = act(alpha * C + beta * C_old + bias[j])        (beta == 0: C_old is not read)

    as the epilogue line of the block-tile loop writes it ("How a Matrix Multiply Runs on a
    GPU", section "Level 2"), bias per column j, the activation applied last: ReLU max(x, 0), or
    GELU x * Phi(x) with Phi the standard normal distribution function (erf form).  S is the
    scale a parity tolerance is normalised by: the magnitudes that enter the activation's
    argument (|alpha| D + |beta C_old| + |bias|), times 1.13, a bound on the slope of either
    activation.
    """
    from scipy.special import erf
    C = np.asarray(C, dtype=np.float64)
    pre = alpha * C
    S = abs(alpha) * np.asarray(D, dtype=np.float64)
    if beta != 0.0:
        old = np.asarray(C_old, dtype=np.float64)
        pre = pre + beta * old
        S = S + np.abs(beta * old)
    if bias is not None:
        b = np.asarray(bias, dtype=np.float64)[None, :]
        pre = pre + b
        S = S + np.abs(b)
    if activation == ACT_RELU:
        Y = np.maximum(pre, 0.0)
    elif activation == ACT_GELU:
        Y = pre * 0.5 * (1.0 + erf(pre / np.sqrt(2.0)))
    elif activation == ACT_NONE:
        Y = pre
    else:
        raise ValueError(f"unknown activation {activation}")
    return Y, 1.13 * S


def _extent(rows, cols, ld, order):
    """Elements a rows x cols matrix spans from its first element."""
    return (rows - 1) * ld + cols if order == 0 else (cols - 1) * ld + rows


def normalised_error(C_test: np.ndarray, C_ref: np.ndarray, D: np.ndarray) -> float:
    """max over elements of |C_test - C_ref| / D.

    Where D == 0 (every product is zero) the test value must be exactly zero (-0 counts
    as zero); a mismatch there, or any NaN / inf in C_test, returns inf.
    """
    C_test = np.asarray(C_test, dtype=np.float64)
    if C_test.size == 0:
        return 0.0
    if not np.all(np.isfinite(C_test)):
        return float("inf")
    diff = np.abs(C_test - C_ref)
    zero = D == 0
    if np.any(diff[zero] != 0):
        return float("inf")
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(zero, 0.0, diff / np.where(zero, 1.0, D))
    return float(rel.max())


def num_threads(lib=None) -> int:
    return int((lib or load()).oracle_num_threads())
