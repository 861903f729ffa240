"""Seeded synthetic inputs for C = A.B, shared by the HIP path's tests/bench and the oracle.

This module holds no GEMM arithmetic.  It only draws operand values, rounds them to
bf16 bit patterns where a workload asks for bf16 inputs, and lays a logical matrix
out in memory per (order, leading dimension).  Both sides of a parity test read the
very same buffers it returns.

Value recipes follow the pages' workloads:
  * square, ragged and skinny shapes use i.i.d. uniform[-1, 1] entries;
  * the LLM linear-layer shapes (the LLaMA-2-7B forward cited in "GEMM Optimization",
    section "1. Why GEMM Matters"; hidden 4096, FFN 11008, 2K tokens) use activations
    ~ N(0, 1) and weights ~ N(0, 0.02) (0.02 read as the standard deviation).
No dataset or trained weights stand behind any of them: the values are synthetic.

bf16 rounding is round-to-nearest-even of the fp32 value, done once here on the host; so is
the rounding to the two OCP 8-bit formats (E4M3, E5M2) of the fp8 workloads ("A06 - Tiled Matrix
Multiply (GEMM)", section "Matrix cores: MFMA and Tensor Cores", names fp8 as a matrix-core input
type; its format is read as the OCP one gfx950's matrix instructions take).  A dtype of "e4m3" or
"e5m2" gives both operands that format; "e4m3_e5m2" and "e5m2_e4m3" name A's and B's.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

ROW_MAJOR = 0
COL_MAJOR = 1


@dataclass(frozen=True)
class Workload:
    """A GEMM problem: shape, input dtype, operand orders and value recipe."""
    name: str
    wid: int                 # small integer mixed into every seed
    M: int
    N: int
    K: int
    dtype: str               # "f32", "bf16", "f16" or an 8-bit pairing of FP8_DTYPES (inputs); C is fp32
    order_a: int = ROW_MAJOR
    order_b: int = ROW_MAJOR
    order_c: int = ROW_MAJOR
    dist: str = "uniform"    # "uniform" -> U[-1,1]; "llm" -> A~N(0,1), B~N(0,0.02); see draw()
    batch: int = 1           # entries of a strided batch (1: one problem)
    layout: tuple = ()       # batched: (("lda", v), ("sa", v), ...) for make_batched_problem

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * self.batch


# The workloads the pages' measurements are about (all synthetic).
WORKLOADS = {
    w.name: w for w in [
        Workload("square256_f32", 1, 256, 256, 256, "f32"),
        Workload("probe16_f32", 1, 16, 16, 16, "f32"),
        Workload("square4096_f32", 2, 4096, 4096, 4096, "f32"),
        Workload("square4096_f32_rc", 2, 4096, 4096, 4096, "f32", ROW_MAJOR, COL_MAJOR),
        Workload("square4096_bf16", 3, 4096, 4096, 4096, "bf16", ROW_MAJOR, COL_MAJOR),
        Workload("square4096_f16", 3, 4096, 4096, 4096, "f16", ROW_MAJOR, COL_MAJOR),
        # PyTorch's `a @ b` layout: both operands row-major (B n-contiguous)
        Workload("square4096_bf16_rr", 3, 4096, 4096, 4096, "bf16"),
        Workload("square4096_e4m3", 3, 4096, 4096, 4096, "e4m3", ROW_MAJOR, COL_MAJOR),
        Workload("square4096_e5m2", 3, 4096, 4096, 4096, "e5m2", ROW_MAJOR, COL_MAJOR),
        Workload("llm_ffn_up_2048x11008x4096_e4m3", 5, 2048, 11008, 4096, "e4m3", ROW_MAJOR, COL_MAJOR, ROW_MAJOR,
                 "llm"),
        Workload("ragged1000_f32", 4, 1000, 1000, 1000, "f32"),
        Workload("ragged1000_bf16", 4, 1000, 1000, 1000, "bf16", ROW_MAJOR, COL_MAJOR),
        Workload("ragged4095x4097x1023_f32", 4, 4095, 4097, 1023, "f32"),
        Workload("ragged4095x4097x1023_bf16", 4, 4095, 4097, 1023, "bf16", ROW_MAJOR, COL_MAJOR),
        Workload("skinny16x4096x4096_f32", 4, 16, 4096, 4096, "f32"),
        Workload("skinny16x4096x4096_bf16", 4, 16, 4096, 4096, "bf16", ROW_MAJOR, COL_MAJOR),
        Workload("llm_attn_proj_2048x4096x4096", 5, 2048, 4096, 4096, "bf16", ROW_MAJOR, COL_MAJOR, ROW_MAJOR, "llm"),
        Workload("llm_ffn_up_2048x11008x4096", 5, 2048, 11008, 4096, "bf16", ROW_MAJOR, COL_MAJOR, ROW_MAJOR, "llm"),
        Workload("llm_ffn_down_2048x4096x11008", 5, 2048, 4096, 11008, "bf16", ROW_MAJOR, COL_MAJOR, ROW_MAJOR, "llm"),
        # one GPU's share of the 4096^3 GEMMs with B and C split by columns over eight GPUs
        # (A replicated): 32 tiles of 256 x 256 for 256 CUs
        Workload("shard4096x512x4096_f32", 8, 4096, 512, 4096, "f32"),
        Workload("shard4096x512x4096_bf16", 8, 4096, 512, 4096, "bf16", ROW_MAJOR, COL_MAJOR),
        # few columns of C and a long K: too few output blocks for the CUs (split-K's case)
        Workload("fewcols16x1024x16384_f32", 6, 16, 1024, 16384, "f32"),
        Workload("fewcols16x1024x16384_bf16", 6, 16, 1024, 16384, "bf16", ROW_MAJOR, COL_MAJOR),
        # few rows and many columns: 16-column blocks of C would take two rounds of the CUs
        Workload("fewrows16x8192x4096_f32", 6, 16, 8192, 4096, "f32"),
        # LLaMA-2-7B attention at 2K tokens, per head (32 heads of 128): the scores Q.K^T and the
        # scores times V as strided batches.  Q, K, V and the output are [tokens, heads, 128]
        # (leading dimension 4096, stride 128 per head); the scores are [heads, 2048, 2048].
        Workload("attn_scores_32x2048x2048x128_bf16", 7, 2048, 2048, 128, "bf16", ROW_MAJOR, COL_MAJOR,
                 ROW_MAJOR, "act", 32, (("lda", 4096), ("sa", 128), ("ldb", 4096), ("sb", 128),
                                        ("ldc", 2048), ("sc", 2048 * 2048))),
        Workload("attn_pv_32x2048x128x2048_bf16", 7, 2048, 128, 2048, "bf16", ROW_MAJOR, ROW_MAJOR,
                 ROW_MAJOR, "probs", 32, (("lda", 2048), ("sa", 2048 * 2048), ("ldb", 4096), ("sb", 128),
                                         ("ldc", 4096), ("sc", 128))),
    ]
}


def rng_for(wid: int, M: int, N: int, K: int, operand: int, extra: int = 0) -> np.random.Generator:
    """PCG64 stream for one operand (0 = A, 1 = B) of one problem."""
    return np.random.default_rng([wid, M, N, K, operand, extra])


def draw(rng: np.random.Generator, rows: int, cols: int, dist: str, operand: int) -> np.ndarray:
    """Logical rows x cols fp32 matrix (row-major in logical order)."""
    if dist == "uniform":
        x = rng.uniform(-1.0, 1.0, (rows, cols))
    elif dist == "llm":
        sigma = 1.0 if operand == 0 else 0.02
        x = rng.standard_normal((rows, cols)) * sigma
    elif dist == "unit":          # [0, 1): the teaching module's lab inputs
        x = rng.uniform(0.0, 1.0, (rows, cols))
    elif dist == "act":           # activations on both sides (attention's Q and K): N(0, 1)
        x = rng.standard_normal((rows, cols))
    elif dist == "probs":         # A: attention probabilities, U[0, 2/cols) (rows sum to ~1); B ~ N(0, 1)
        x = rng.uniform(0.0, 2.0 / cols, (rows, cols)) if operand == 0 else rng.standard_normal((rows, cols))
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return x.astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bit patterns.

    NaN stays NaN (quiet); finite values that round past the largest bf16 become inf,
    as IEEE rounding prescribes.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    # uint32 arithmetic: only NaN patterns (>= 0xFFFF8000) can wrap, and they are replaced below
    rounded = ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if nan.any():
        rounded = rounded.copy()
        rounded[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return rounded


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# OCP 8-bit formats: (exponent bits, fraction bits, bias)
FP8_FORMATS = {"e4m3": (4, 3, 7), "e5m2": (5, 2, 15)}
FP8_DTYPES = {"e4m3": ("e4m3", "e4m3"), "e5m2": ("e5m2", "e5m2"), "e4m3_e5m2": ("e4m3", "e5m2"),
              "e5m2_e4m3": ("e5m2", "e4m3")}


def f32_to_fp8_bits(x: np.ndarray, fmt: str) -> np.ndarray:
    """Round fp32 to an OCP 8-bit format (round to nearest, ties to even); uint8 bit patterns.

    Values that round past the largest finite one become NaN in E4M3 (it has no infinities;
    0x7F) and infinity in E5M2 (0x7C, sign kept); NaN becomes 0x7F in both.
    """
    ebits, mbits, bias = FP8_FORMATS[fmt]
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    finite = np.isfinite(a)
    a = np.where(finite, a, 0.0)
    emin = 1 - bias                                   # exponent of the smallest normal value
    _, e = np.frexp(a)                                # a = m 2^e, m in [0.5, 1)
    E = np.maximum(e - 1, emin)                       # subnormals share the smallest exponent
    q = np.rint(a / np.exp2(E - mbits))               # significand in last-place units, ties to even
    carry = q >= 2 ** (mbits + 1)
    E = np.where(carry, E + 1, E)
    q = np.where(carry, q / 2, q)
    normal = q >= 2 ** mbits
    expf = np.where(normal, E + bias, 0).astype(np.int64)
    frac = np.where(normal, q - 2 ** mbits, q).astype(np.int64)
    bits = (expf << mbits) | frac
    if fmt == "e4m3":
        over = (expf > 15) | ((expf == 15) & (frac == 7)) | np.isinf(x)
        bits = np.where(over, 0x7F, bits)
    else:
        over = (expf >= 31) | np.isinf(x)
        bits = np.where(over, 0x7C, bits)
    sign = np.signbit(x).astype(np.int64) << 7
    bits = np.where(np.isnan(x), 0x7F, bits | sign)
    return bits.astype(np.uint8)


def fp8_bits_to_f32(b: np.ndarray, fmt: str) -> np.ndarray:
    """Exact widening of OCP 8-bit bit patterns to fp32 (every such value is an fp32 value)."""
    ebits, mbits, bias = FP8_FORMATS[fmt]
    table = np.empty(256, dtype=np.float64)
    for v in range(256):
        sign = -1.0 if v >> 7 else 1.0
        expf, frac = (v >> mbits) & ((1 << ebits) - 1), v & ((1 << mbits) - 1)
        top = (1 << ebits) - 1
        if fmt == "e4m3" and expf == top and frac == (1 << mbits) - 1:
            table[v] = np.nan
        elif fmt == "e5m2" and expf == top:
            table[v] = sign * np.inf if frac == 0 else np.nan
        elif expf == 0:
            table[v] = sign * frac * 2.0 ** (1 - bias - mbits)
        else:
            table[v] = sign * (1 + frac / 2 ** mbits) * 2.0 ** (expf - bias)
    return table[np.asarray(b, dtype=np.uint8)].astype(np.float32)


def lay_out(logical: np.ndarray, order: int, ld: int | None = None) -> tuple[np.ndarray, int]:
    """Place a logical R x C matrix in a flat buffer with the given order and leading dim.

    Row-major: element (r, c) at r*ld + c, ld >= C.  Column-major: at r + c*ld, ld >= R.
    Padding slots (ld beyond the minimum) hold a sentinel so that a kernel reading them
    produces visibly wrong results.  Returns (flat buffer, ld).
    """
    R, C = logical.shape
    if order == ROW_MAJOR:
        ld = C if ld is None else ld
        assert ld >= max(1, C)
        buf = np.full((max(R, 0), ld), _sentinel(logical.dtype), dtype=logical.dtype)
        buf[:, :C] = logical
        flat = buf.reshape(-1)
    else:
        ld = R if ld is None else ld
        assert ld >= max(1, R)
        buf = np.full((max(C, 0), ld), _sentinel(logical.dtype), dtype=logical.dtype)
        buf[:, :R] = logical.T
        flat = buf.reshape(-1)
    if flat.size == 0:
        flat = np.zeros(1, dtype=logical.dtype)   # never read; keeps pointers non-null
    return flat, ld


def _sentinel(dtype) -> object:
    if dtype == np.uint8:
        return np.uint8(0x7F)        # NaN in both 8-bit formats
    if dtype == np.uint16:
        return np.uint16(0x7FC1)     # a bf16 NaN
    if dtype == np.float16:
        return np.float16(np.nan)
    return np.float32(np.nan)


@dataclass
class Problem:
    """One seeded problem: logical operands plus their laid-out buffers."""
    M: int
    N: int
    K: int
    dtype: str
    order_a: int
    order_b: int
    order_c: int
    A_logical: np.ndarray    # fp32 (M, K), uint16 bf16 bits (M, K) or float16 (M, K)
    B_logical: np.ndarray
    A: np.ndarray            # flat buffer
    lda: int
    B: np.ndarray
    ldb: int
    ldc: int

    def a_f32(self) -> np.ndarray:
        return _to_f32(self.A_logical, self.dtype, 0)

    def b_f32(self) -> np.ndarray:
        return _to_f32(self.B_logical, self.dtype, 1)

    @property
    def fmt_a(self):
        """A's 8-bit format ("e4m3" / "e5m2"), None for other input types."""
        return FP8_DTYPES[self.dtype][0] if self.dtype in FP8_DTYPES else None

    @property
    def fmt_b(self):
        return FP8_DTYPES[self.dtype][1] if self.dtype in FP8_DTYPES else None


def oracle_formats(p) -> dict:
    """The fmt_a / fmt_b arguments the oracle needs for a problem's 8-bit operands ({} otherwise)."""
    return {"fmt_a": p.fmt_a, "fmt_b": p.fmt_b} if p.dtype in FP8_DTYPES else {}


def _to_f32(x: np.ndarray, dtype: str, operand: int = 0) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f32(x)
    if dtype in FP8_DTYPES:
        return fp8_bits_to_f32(x, FP8_DTYPES[dtype][operand])
    return x.astype(np.float32) if dtype == "f16" else x


def make_problem(M: int, N: int, K: int, dtype: str = "f32", order_a: int = ROW_MAJOR,
                 order_b: int = ROW_MAJOR, order_c: int = ROW_MAJOR, dist: str = "uniform",
                 wid: int = 0, pad_a: int = 0, pad_b: int = 0, pad_c: int = 0,
                 A_logical: np.ndarray | None = None, B_logical: np.ndarray | None = None) -> Problem:
    """Draw (or take) logical A (M x K) and B (K x N) and lay them out.

    pad_* adds that many slots to the minimum leading dimension.
    A_logical / B_logical, if given, are fp32 matrices used instead of random draws
    (rounded to bf16 when dtype == "bf16", to fp16 when "f16": numpy's round to nearest
    even, values beyond the fp16 range becoming inf).
    """
    if A_logical is None:
        A_logical = draw(rng_for(wid, M, N, K, 0), M, K, dist, 0)
    if B_logical is None:
        B_logical = draw(rng_for(wid, M, N, K, 1), K, N, dist, 1)
    A_logical = np.asarray(A_logical, dtype=np.float32).reshape(M, K)
    B_logical = np.asarray(B_logical, dtype=np.float32).reshape(K, N)
    if dtype == "bf16":
        A_logical = f32_to_bf16_bits(A_logical)
        B_logical = f32_to_bf16_bits(B_logical)
    elif dtype == "f16":
        A_logical = A_logical.astype(np.float16)
        B_logical = B_logical.astype(np.float16)
    elif dtype in FP8_DTYPES:
        A_logical = f32_to_fp8_bits(A_logical, FP8_DTYPES[dtype][0])
        B_logical = f32_to_fp8_bits(B_logical, FP8_DTYPES[dtype][1])
    elif dtype != "f32":
        raise ValueError(dtype)
    lda0 = K if order_a == ROW_MAJOR else M
    ldb0 = N if order_b == ROW_MAJOR else K
    ldc0 = N if order_c == ROW_MAJOR else M
    A, lda = lay_out(A_logical, order_a, max(1, lda0) + pad_a)
    B, ldb = lay_out(B_logical, order_b, max(1, ldb0) + pad_b)
    return Problem(M, N, K, dtype, order_a, order_b, order_c, A_logical, B_logical,
                   A, lda, B, ldb, max(1, ldc0) + pad_c)


@dataclass
class BatchedProblem:
    """A seeded strided batch: batch entries of one M x N x K shape in shared flat buffers.

    Entry z's element (r, c) of an operand sits at z*stride + offset(r, c) (offset by the
    operand's order and leading dimension).  A stride of 0 for A or B means one matrix for
    every entry (its logical array repeats).  Slots no entry uses hold the sentinel.
    """
    batch: int
    M: int
    N: int
    K: int
    dtype: str
    order_a: int
    order_b: int
    order_c: int
    A_logical: np.ndarray    # (batch, M, K) in the input encoding
    B_logical: np.ndarray    # (batch, K, N)
    A: np.ndarray
    lda: int
    sa: int
    B: np.ndarray
    ldb: int
    sb: int
    ldc: int
    sc: int

    def c_size(self) -> int:
        return self.sc * (self.batch - 1) + _whole(self.M, self.N, self.ldc, self.order_c) \
            if self.batch and self.M and self.N else 1

    def c_view(self, flat: np.ndarray) -> np.ndarray:
        """(batch, M, N) strided view of the entries in a C buffer."""
        return entry_view(flat, self.batch, self.M, self.N, self.ldc, self.sc, self.order_c)

    def c_untouched(self, flat: np.ndarray) -> np.ndarray:
        """Values of the C slots that belong to no entry."""
        mask = np.ones(flat.size, dtype=bool)
        entry_view(mask, self.batch, self.M, self.N, self.ldc, self.sc, self.order_c)[...] = False
        return flat[mask]


def _span(R: int, C: int, ld: int, order: int) -> int:
    return (R - 1) * ld + C if order == ROW_MAJOR else (C - 1) * ld + R


def _whole(R: int, C: int, ld: int, order: int) -> int:
    """Elements of an R x C matrix stored in whole rows (columns) of ld, as lay_out stores one."""
    return R * ld if order == ROW_MAJOR else C * ld


def entries_disjoint(batch: int, R: int, C: int, ld: int, stride: int, order: int) -> bool:
    """Entries one after another (stride >= span) or side by side within ld."""
    if batch <= 1:
        return True
    inner = C if order == ROW_MAJOR else R
    return stride >= _span(R, C, ld, order) or (stride >= inner and (batch - 1) * stride + inner <= ld)


def entry_view(flat: np.ndarray, batch: int, R: int, C: int, ld: int, stride: int, order: int) -> np.ndarray:
    """(batch, R, C) view of flat: entry z's element (r, c) at z*stride + offset(r, c)."""
    if batch == 0 or R == 0 or C == 0:
        return np.zeros((batch, R, C), dtype=flat.dtype)
    assert flat.size >= stride * (batch - 1) + _span(R, C, ld, order)
    e = flat.itemsize
    strides = (stride * e, ld * e, e) if order == ROW_MAJOR else (stride * e, e, ld * e)
    return np.lib.stride_tricks.as_strided(flat, shape=(batch, R, C), strides=strides)


def _place(logical: np.ndarray, order: int, ld: int, stride: int) -> np.ndarray:
    batch, R, C = logical.shape
    if batch == 0 or R == 0 or C == 0:
        return np.zeros(1, dtype=logical.dtype)
    assert stride == 0 or entries_disjoint(batch, R, C, ld, stride, order), "entries of this layout overlap"
    # the last entry ends with whole rows (columns) of ld, as a single laid-out matrix does
    flat = np.full(stride * (batch - 1) + _whole(R, C, ld, order), _sentinel(logical.dtype), dtype=logical.dtype)
    entry_view(flat, batch, R, C, ld, stride, order)[...] = logical
    return flat


def make_batched_problem(batch: int, M: int, N: int, K: int, dtype: str = "f32", order_a: int = ROW_MAJOR,
                         order_b: int = ROW_MAJOR, order_c: int = ROW_MAJOR, lda: int | None = None,
                         sa: int | None = None, ldb: int | None = None, sb: int | None = None,
                         ldc: int | None = None, sc: int | None = None, dist: str = "uniform",
                         wid: int = 0, A_logical: np.ndarray | None = None,
                         B_logical: np.ndarray | None = None) -> BatchedProblem:
    """Draw (or take, as fp32 (batch, rows, cols) arrays) every entry's operands and lay them out.

    Leading dimensions default to tight, strides to one tight entry after another.  Entry z
    draws from its own seeded stream; with stride 0 entry 0's matrix serves all.
    """
    lda = lda if lda is not None else max(1, K if order_a == ROW_MAJOR else M)
    ldb = ldb if ldb is not None else max(1, N if order_b == ROW_MAJOR else K)
    ldc = ldc if ldc is not None else max(1, N if order_c == ROW_MAJOR else M)
    sa = sa if sa is not None else _span(M, K, lda, order_a) if M and K else 0
    sb = sb if sb is not None else _span(K, N, ldb, order_b) if K and N else 0
    sc = sc if sc is not None else _span(M, N, ldc, order_c) if M and N else 0

    def operand(given, rows, cols, operand_id, stride):
        if given is not None:
            x = np.asarray(given, dtype=np.float32).reshape(batch, rows, cols)
        else:
            n = batch if stride else min(batch, 1)
            x = np.stack([draw(rng_for(wid, M, N, K, operand_id, z + 1), rows, cols, dist, operand_id)
                          for z in range(n)]) if n else np.zeros((0, rows, cols), np.float32)
            if not stride and batch:
                x = np.repeat(x, batch, axis=0)
        if dtype == "bf16":
            return f32_to_bf16_bits(x.reshape(-1)).reshape(x.shape)
        if dtype == "f16":
            return x.astype(np.float16)
        if dtype != "f32":
            raise ValueError(dtype)
        return x

    A_log = operand(A_logical, M, K, 0, sa)
    B_log = operand(B_logical, K, N, 1, sb)
    return BatchedProblem(batch, M, N, K, dtype, order_a, order_b, order_c, A_log, B_log,
                          _place(A_log, order_a, lda, sa), lda, sa, _place(B_log, order_b, ldb, sb), ldb, sb,
                          ldc, sc)


def workload_problem(name: str, seed_offset: int = 0, K: int | None = None):
    """The named workload's seeded inputs: a Problem, or a BatchedProblem for a batch.  K, if
    given, replaces the workload's depth (same recipe otherwise)."""
    w = WORKLOADS[name] if K is None else dataclasses.replace(WORKLOADS[name], K=K)
    if w.batch > 1:
        return make_batched_problem(w.batch, w.M, w.N, w.K, w.dtype, w.order_a, w.order_b, w.order_c,
                                    dist=w.dist, wid=w.wid + seed_offset, **dict(w.layout))
    return make_problem(w.M, w.N, w.K, w.dtype, w.order_a, w.order_b, w.order_c, w.dist, w.wid + seed_offset)


def unpack_c(flat: np.ndarray, M: int, N: int, ldc: int, order_c: int) -> np.ndarray:
    """Logical M x N view of a C buffer laid out with (ldc, order_c)."""
    if order_c == ROW_MAJOR:
        return flat.reshape(-1, ldc)[:M, :N] if M and N else np.zeros((M, N), flat.dtype)
    return flat.reshape(-1, ldc)[:N, :M].T if M and N else np.zeros((M, N), flat.dtype)


def c_buffer_size(M: int, N: int, ldc: int, order_c: int) -> int:
    if M == 0 or N == 0:
        return 1
    return (M * ldc) if order_c == ROW_MAJOR else (N * ldc)
