"""GPU parity of gemm_fp8_f32acc (OCP E4M3 / E5M2 inputs, FP32 accumulate) against the fp64 oracle.

The oracle decodes each byte from its sign, exponent and fraction fields; every product of two
decoded values is exact in FP32, so the bar is the one for the 16-bit inputs: normalised error
<= 1e-4 for random values, bit-exact where any summation order is exact (small integers,
permutations, identities, single products of the largest finite values and of subnormals).
"""
import numpy as np
import pytest

import gemm_f32_amd as g
import gemm_inputs as gi
import oracle
from gemm_inputs import COL_MAJOR, ROW_MAJOR
from gpu_util import FP8_CODE, TOL, check, logical_c, run, to_device

pytestmark = pytest.mark.gpu

PAIRS = ["e4m3", "e5m2", "e4m3_e5m2", "e5m2_e4m3"]
OC = [ROW_MAJOR, COL_MAJOR]
OC_IDS = ["RCR", "RCC"]

# whole tiles, several tiles with a K tail, ragged M and N, K below one k-tile (128) and below one
# 16-byte chunk (16), one element
SHAPES = [(256, 256, 128), (512, 384, 256), (300, 264, 192), (1000, 260, 1023), (257, 385, 65),
          (33, 300, 127), (1, 1, 1), (5, 300, 7), (130, 200, 16), (520, 392, 640)]


@pytest.mark.parametrize("oc", OC, ids=OC_IDS)
@pytest.mark.parametrize("dtype", PAIRS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fp8_random(dtype, oc, shape):
    M, N, K = shape
    p = gi.make_problem(M, N, K, dtype, ROW_MAJOR, COL_MAJOR, oc, wid=70)
    check(p, key=("fp8", dtype, oc, shape))
    assert g.gemm_last_kernel().startswith("fp8_dma")


@pytest.mark.parametrize("dtype", PAIRS)
def test_fp8_both_tiles_run(dtype):
    """A C of more than one round of 256 x 128 tiles takes 256 x 256 tiles, a small one 256 x 128;
    both against the oracle."""
    for shape, name in [((4096, 2304, 256), "fp8_dma256x256"), ((256, 128, 384), "fp8_dma256x128")]:
        p = gi.make_problem(*shape, dtype, ROW_MAJOR, COL_MAJOR, wid=71)
        check(p)
        assert g.gemm_last_kernel() == name


@pytest.mark.parametrize("dtype", PAIRS)
@pytest.mark.parametrize("shape", [(520, 392, 640), (300, 257, 129), (64, 64, 16), (130, 200, 5)],
                         ids=lambda s: "x".join(map(str, s)))
def test_fp8_small_integer_exact(dtype, shape):
    """Integers in [-4, 4] are exact in both formats and every sum is exact in FP32."""
    M, N, K = shape
    rng = np.random.default_rng(M + 5 * N + K)
    A = rng.integers(-4, 5, (M, K)).astype(np.float32)
    B = rng.integers(-4, 5, (K, N)).astype(np.float32)
    p = gi.make_problem(M, N, K, dtype, ROW_MAJOR, COL_MAJOR, A_logical=A, B_logical=B)
    check(p, exact=True)


@pytest.mark.parametrize("dtype", PAIRS)
@pytest.mark.parametrize("oc", OC, ids=OC_IDS)
def test_fp8_closed_forms(dtype, oc):
    """A = permutation gives B's rows, B = permutation gives A's columns, bit for bit; ones
    give K.  A transposed operand or a wrong pairing of k between A and B fails these."""
    n = 384
    perm = np.random.default_rng(7).permutation(n)
    P = np.eye(n, dtype=np.float32)[perm]
    R = np.random.default_rng(8).uniform(-1, 1, (n, n)).astype(np.float32)
    pb = gi.make_problem(n, n, n, dtype, ROW_MAJOR, COL_MAJOR, oc, A_logical=P, B_logical=R)
    assert np.array_equal(logical_c(pb, run(pb)), pb.b_f32()[perm])
    pa = gi.make_problem(n, n, n, dtype, ROW_MAJOR, COL_MAJOR, oc, A_logical=R, B_logical=P.T.copy())
    assert np.array_equal(logical_c(pa, run(pa)), pa.a_f32()[:, perm])
    K = 1000
    ones = gi.make_problem(300, 260, K, dtype, ROW_MAJOR, COL_MAJOR, oc, A_logical=np.ones((300, K)),
                           B_logical=np.ones((K, 260)))
    assert np.all(logical_c(ones, run(ones)) == K)


@pytest.mark.parametrize("dtype", PAIRS)
def test_fp8_extreme_values(dtype):
    """Single products of the largest finite values, of the smallest subnormals and of signed
    zeros, each alone in its output: exact in FP32, so C must equal the oracle bit for bit."""
    fa, fb = gi.FP8_DTYPES[dtype]
    big = {"e4m3": 448.0, "e5m2": 57344.0}
    tiny = {"e4m3": 2.0 ** -9, "e5m2": 2.0 ** -16}
    M, N, K = 256, 256, 256
    A = np.zeros((M, K), np.float32)
    B = np.zeros((K, N), np.float32)
    for i in range(0, M, 4):
        k, m = (7 * i) % K, (i // 4) % 5
        A[i, k] = [big[fa], -big[fa], tiny[fa], -tiny[fa], tiny[fa]][m]
        B[k, (3 * i) % N] = [big[fb], tiny[fb], -big[fb], -0.0, tiny[fb]][m]
    p = gi.make_problem(M, N, K, dtype, ROW_MAJOR, COL_MAJOR, A_logical=A, B_logical=B)
    C = logical_c(p, run(p))
    ref, _ = oracle.gemm(M, N, K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b, **gi.oracle_formats(p))
    assert np.array_equal(C.astype(np.float64), ref)
    assert np.any(np.abs(C) == big[fa] * big[fb]) and np.any(np.abs(C) == tiny[fa] * tiny[fb])


@pytest.mark.parametrize("dtype", ["e4m3", "e5m2"])
def test_fp8_non_finite_inputs(dtype):
    """A NaN in A makes its row of C NaN (NaN times anything, zero included, is NaN); an E5M2
    infinity times a positive B column gives +inf there; every other entry stays exact."""
    M, N, K = 256, 256, 256
    rng = np.random.default_rng(3)
    A = rng.integers(-3, 4, (M, K)).astype(np.float32)
    B = rng.integers(0, 3, (K, N)).astype(np.float32)
    B[5, :] = 1.0
    p = gi.make_problem(M, N, K, dtype, ROW_MAJOR, COL_MAJOR, A_logical=A, B_logical=B)
    Ab = p.A.reshape(M, p.lda)          # row-major A: row i, column k at i * lda + k
    Ab[17, 5] = 0x7F                     # NaN in both formats (E4M3 S.1111.111, E5M2 S.11111.11)
    if dtype == "e5m2":
        Ab[40, 5] = 0x7C                 # +inf
    C = logical_c(p, run(p))
    assert np.all(np.isnan(C[17]))
    if dtype == "e5m2":
        assert np.all(np.isposinf(C[40]))
    rest = [i for i in range(M) if i not in (17, 40)]
    assert np.array_equal(C[rest], (A @ B)[rest])


@pytest.mark.parametrize("oc", OC, ids=OC_IDS)
@pytest.mark.parametrize("pad", [1, 3, 8])
def test_fp8_padded_byte_aligned_rows(oc, pad):
    """Odd leading dimensions put rows at odd byte addresses; padding bytes hold NaN (0x7F), so a
    kernel that reads them poisons C."""
    p = gi.make_problem(300, 260, 200, "e4m3_e5m2", ROW_MAJOR, COL_MAJOR, oc, wid=72, pad_a=pad, pad_b=pad,
                        pad_c=pad)
    check(p)


@pytest.mark.parametrize("K", [1, 3, 8, 15, 16, 17, 31, 63, 127, 129, 255])
def test_fp8_k_tails(K):
    p = gi.make_problem(300, 270, K, "e4m3", ROW_MAJOR, COL_MAJOR, wid=73)
    check(p)


def test_fp8_k_zero_and_empty():
    p = gi.make_problem(37, 45, 0, "e4m3", ROW_MAJOR, COL_MAJOR, pad_c=3)
    C = logical_c(p, run(p))
    assert np.all(C == 0) and g.gemm_last_kernel() == "zero_c"
    e = gi.make_problem(0, 5, 7, "e5m2", ROW_MAJOR, COL_MAJOR)
    assert np.all(np.isnan(run(e)))


def test_fp8_repeated_runs_identical():
    p = gi.make_problem(777, 1025, 513, "e4m3", ROW_MAJOR, COL_MAJOR, wid=74)
    A, B = to_device(p.A), to_device(p.B)
    first = run(p, A=A, B=B)
    for _ in range(5):
        assert np.array_equal(run(p, A=A, B=B), first, equal_nan=True)


@pytest.mark.parametrize("dtype", ["e4m3", "e5m2"])
def test_fp8_square4096_sampled(dtype):
    """The 4096^3 problem the benchmark times: 2048 sampled outputs against the oracle."""
    n = 4096
    p = gi.make_problem(n, n, n, dtype, ROW_MAJOR, COL_MAJOR, wid=3)
    C = logical_c(p, run(p))
    rng = np.random.default_rng(11)
    rows, cols = rng.integers(0, n, 2048), rng.integers(0, n, 2048)
    ref, D = oracle.gemm_sampled(n, n, n, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b, rows, cols,
                                 **gi.oracle_formats(p))
    err = oracle.normalised_error(C[rows, cols], ref, D)
    assert err <= TOL[dtype], f"normalised error {err:.3e}"
    assert g.gemm_last_kernel() == "fp8_dma256x256"


def test_fp8_rejects_other_layouts():
    p = gi.make_problem(64, 64, 64, "e4m3", ROW_MAJOR, COL_MAJOR)
    A, B = to_device(p.A), to_device(p.B)
    import torch
    C = torch.zeros(64 * 64, dtype=torch.float32, device="cuda")
    for oa, ob in [(COL_MAJOR, COL_MAJOR), (ROW_MAJOR, ROW_MAJOR), (COL_MAJOR, ROW_MAJOR)]:
        with pytest.raises(g.GemmError) as e:
            g.gemm_fp8_f32acc(64, 64, 64, A.data_ptr(), 64, oa, FP8_CODE["e4m3"], B.data_ptr(), 64, ob,
                              FP8_CODE["e4m3"], C.data_ptr(), 64, ROW_MAJOR, 0)
        assert e.value.status == g.Status.ERR_INVALID_VALUE
    torch.cuda.synchronize()
    assert torch.count_nonzero(C).item() == 0
