"""Helpers for the GPU parity tests: run one problem through libgemm's C ABI and compare
with the fp64 oracle on the same seeded buffers."""
from __future__ import annotations

import functools

import numpy as np

import gemm_f32_amd as g
import gemm_inputs as gi
import oracle

# max |C - C_ref| / sum_k |A_ik B_kj|; fp16 and 8-bit inputs, like bf16, give exact products in
# FP32, so only the FP32 sums round
TOL = {"f32": 1e-5, "bf16": 1e-4, "f16": 1e-4, **{d: 1e-4 for d in gi.FP8_DTYPES}}
FP8_CODE = {"e4m3": g.Fp8.E4M3, "e5m2": g.Fp8.E5M2}


def to_device(buf: np.ndarray):
    import torch
    if buf.dtype in (np.uint16, np.float16):
        buf = buf.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(buf)).to("cuda")


def run(p: gi.Problem, algo=g.Algo.AUTO, A=None, B=None):
    """C buffer (flat, float32 numpy) after one libgemm call; C starts as NaN everywhere."""
    import torch
    A = to_device(p.A) if A is None else A
    B = to_device(p.B) if B is None else B
    n = gi.c_buffer_size(p.M, p.N, p.ldc, p.order_c)
    C = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    print(f"[gpu] {p.dtype} algo={int(algo)} M={p.M} N={p.N} K={p.K} orders=({p.order_a},"
          f"{p.order_b},{p.order_c}) ld=({p.lda},{p.ldb},{p.ldc})", flush=True)
    stream = torch.cuda.current_stream().cuda_stream
    if p.dtype in gi.FP8_DTYPES:           # one kernel family: no algorithm argument
        g.gemm_fp8_f32acc(p.M, p.N, p.K, A.data_ptr(), p.lda, p.order_a, FP8_CODE[p.fmt_a], B.data_ptr(), p.ldb,
                          p.order_b, FP8_CODE[p.fmt_b], C.data_ptr(), p.ldc, p.order_c, stream)
    else:
        fn = {"f32": g.gemm_f32_algo, "bf16": g.gemm_bf16_f32acc_algo, "f16": g.gemm_f16_f32acc_algo}[p.dtype]
        fn(algo, p.M, p.N, p.K, A.data_ptr(), p.lda, p.order_a, B.data_ptr(), p.ldb, p.order_b,
           C.data_ptr(), p.ldc, p.order_c, stream)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def logical_c(p: gi.Problem, flat: np.ndarray) -> np.ndarray:
    return gi.unpack_c(flat, p.M, p.N, p.ldc, p.order_c)


def padding_untouched(p: gi.Problem, flat: np.ndarray) -> bool:
    """Slots of C beyond the logical matrix (ldc padding) still hold the NaN fill."""
    if p.M == 0 or p.N == 0:
        return bool(np.all(np.isnan(flat)))
    inner = p.N if p.order_c == gi.ROW_MAJOR else p.M
    return bool(np.all(np.isnan(flat.reshape(-1, p.ldc)[:, inner:])))


@functools.lru_cache(maxsize=64)
def _oracle_cached(key):
    p = _PROBLEMS[key]
    return oracle.gemm(p.M, p.N, p.K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b, **gi.oracle_formats(p))


_PROBLEMS: dict = {}


def reference(p: gi.Problem, key=None):
    """(C_ref, D) from the oracle; cached per key when one is given."""
    if key is None:
        return oracle.gemm(p.M, p.N, p.K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b, **gi.oracle_formats(p))
    _PROBLEMS[key] = p
    return _oracle_cached(key)


def check(p: gi.Problem, algo=g.Algo.AUTO, key=None, exact=False):
    """Run and compare element by element; returns the normalised error."""
    flat = run(p, algo)
    C = logical_c(p, flat)
    ref, D = reference(p, key)
    assert padding_untouched(p, flat), "C written outside the logical matrix"
    if exact:
        assert np.array_equal(C.astype(np.float64), ref), "expected a bit-exact result"
        return 0.0
    err = oracle.normalised_error(C, ref, D)
    assert err <= TOL[p.dtype], f"normalised error {err:.3e} > {TOL[p.dtype]:.0e}"
    return err


def run_batched(p: gi.BatchedProblem):
    """C buffer (flat float32 numpy, NaN-filled before the call) after one strided batched call."""
    import torch
    A, B = to_device(p.A), to_device(p.B)
    C = torch.full((p.c_size(),), float("nan"), dtype=torch.float32, device="cuda")
    fn = {"f32": g.gemm_f32_strided_batched, "bf16": g.gemm_bf16_f32acc_strided_batched,
          "f16": g.gemm_f16_f32acc_strided_batched}[p.dtype]
    print(f"[gpu] batched {p.dtype} batch={p.batch} M={p.M} N={p.N} K={p.K} orders=({p.order_a},{p.order_b},"
          f"{p.order_c}) ld=({p.lda},{p.ldb},{p.ldc}) strides=({p.sa},{p.sb},{p.sc})", flush=True)
    fn(p.batch, p.M, p.N, p.K, A.data_ptr(), p.lda, p.sa, p.order_a, B.data_ptr(), p.ldb, p.sb, p.order_b,
       C.data_ptr(), p.ldc, p.sc, p.order_c, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def check_batched(p: gi.BatchedProblem):
    """Run a strided batch and compare every entry element by element with the oracle."""
    flat = run_batched(p)
    assert np.all(np.isnan(p.c_untouched(flat))), "C written outside the entries"
    got = p.c_view(flat)
    ref, D = oracle.gemm_strided_batched(p.batch, p.M, p.N, p.K, p.A, p.lda, p.sa, p.order_a, p.B, p.ldb, p.sb,
                                         p.order_b)
    err = oracle.normalised_error(got, ref, D)
    assert err <= TOL[p.dtype], f"normalised error {err:.3e} > {TOL[p.dtype]:.0e}"
    return err
