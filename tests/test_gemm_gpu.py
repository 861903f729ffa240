"""GPU parity: every libgemm kernel against the fp64 oracle on the same seeded inputs.

Tolerance: max over C of |C_gpu - C_ref| / sum_k |A_ik B_kj|  <=  1e-5 (FP32) and
<= 1e-4 (BF16 inputs, FP32 accumulate).  Closed-form and small-integer cases must be
bit-exact, because any summation order gives the exact result there.
"""
import numpy as np
import pytest

import gemm_f32_amd as g
import gemm_inputs as gi
import oracle
from gemm_inputs import COL_MAJOR, ROW_MAJOR
from gpu_util import TOL, check, logical_c, padding_untouched, reference, run, to_device

pytestmark = pytest.mark.gpu

F32_ALGOS = [g.Algo.NAIVE_UNCOALESCED, g.Algo.NAIVE, g.Algo.TILED, g.Algo.REGBLOCK,
             g.Algo.MFMA_128x128, g.Algo.MFMA_64x64, g.Algo.AUTO]
BF16_ALGOS = [g.Algo.MFMA_256x128, g.Algo.MFMA_128x128, g.Algo.MFMA_64x64, g.Algo.AUTO]
CASES = [("f32", a) for a in F32_ALGOS] + [("bf16", a) for a in BF16_ALGOS]
CASE_IDS = [f"{d}-{a.name}" for d, a in CASES]
ORDERS3 = [(a, b, c) for a in (ROW_MAJOR, COL_MAJOR) for b in (ROW_MAJOR, COL_MAJOR)
           for c in (ROW_MAJOR, COL_MAJOR)]


# --- closed forms at the pages' 16 x 16 x 16 worked size and beyond ---------------------
@pytest.mark.parametrize("dtype,algo", CASES, ids=CASE_IDS)
@pytest.mark.parametrize("n", [16, 64, 129])
def test_closed_forms(dtype, algo, n):
    ones = gi.make_problem(n, n, n, dtype, A_logical=np.ones((n, n)), B_logical=np.ones((n, n)))
    C = logical_c(ones, run(ones, algo))
    assert np.all(C == n), "A = B = ones must give C = K"
    ident = gi.make_problem(n, n, n, dtype, wid=31, A_logical=np.eye(n))
    C = logical_c(ident, run(ident, algo))
    assert np.array_equal(C, ident.b_f32()), "A = I must reproduce B bit for bit"
    perm = np.random.default_rng(n).permutation(n)
    P = np.zeros((n, n)); P[np.arange(n), perm] = 1.0
    pb = gi.make_problem(n, n, n, dtype, wid=32, B_logical=P)
    C = logical_c(pb, run(pb, algo))
    assert np.array_equal(C, pb.a_f32()[:, np.argsort(perm)]), "B = P must permute columns of A"
    pa = gi.make_problem(n, n, n, dtype, wid=33, A_logical=P)
    C = logical_c(pa, run(pa, algo))
    assert np.array_equal(C, pa.b_f32()[perm]), "A = P must permute rows of B"


# --- small integers: exact under any summation order, so GPU == oracle bit for bit ------
@pytest.mark.parametrize("dtype,algo", CASES, ids=CASE_IDS)
@pytest.mark.parametrize("shape", [(64, 64, 64), (300, 257, 129), (33, 517, 1000)],
                         ids=lambda s: "x".join(map(str, s)))
def test_small_integer_exact(dtype, algo, shape):
    M, N, K = shape
    rng = np.random.default_rng(M * 7 + N)
    A = rng.integers(-4, 5, (M, K)).astype(np.float32)
    B = rng.integers(-4, 5, (K, N)).astype(np.float32)
    p = gi.make_problem(M, N, K, dtype, A_logical=A, B_logical=B)
    check(p, algo, exact=True)


# --- random inputs, every order combination, ragged shapes ------------------------------
SHAPES = [(1, 1, 1), (256, 256, 256), (257, 259, 65), (5, 300, 7), (300, 5, 1000),
          (129, 67, 300)]


@pytest.mark.parametrize("dtype,algo", CASES, ids=CASE_IDS)
@pytest.mark.parametrize("orders", ORDERS3, ids=lambda o: "".join("RC"[x] for x in o))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_parity_random(dtype, algo, orders, shape):
    M, N, K = shape
    p = gi.make_problem(M, N, K, dtype, *orders, wid=40)
    check(p, algo, key=("rand", dtype, orders, shape))


# --- the teaching module's boundary trio: only a ragged K exposes a missing zero fill ---
@pytest.mark.parametrize("dtype,algo", CASES, ids=CASE_IDS)
@pytest.mark.parametrize("shape", [(1024, 1024, 1024), (1000, 700, 1024), (1000, 700, 1000)],
                         ids=lambda s: "x".join(map(str, s)))
def test_boundary_trio(dtype, algo, shape):
    if algo in (g.Algo.NAIVE_UNCOALESCED,) and shape[0] > 512:
        pytest.skip("uncoalesced rung is slow; covered at the smaller shapes")
    M, N, K = shape
    oa, ob = (ROW_MAJOR, ROW_MAJOR) if dtype == "f32" else (ROW_MAJOR, COL_MAJOR)
    p = gi.make_problem(M, N, K, dtype, oa, ob, dist="unit", wid=41)
    check(p, algo, key=("trio", dtype, shape))


# --- K below the tile depth, K = 0, empty outputs ---------------------------------------
@pytest.mark.parametrize("dtype,algo", CASES, ids=CASE_IDS)
@pytest.mark.parametrize("K", [1, 3, 8, 15, 31, 63])
def test_k_below_tile(dtype, algo, K):
    p = gi.make_problem(130, 200, K, dtype, ROW_MAJOR, COL_MAJOR if dtype == "bf16" else ROW_MAJOR, wid=42)
    check(p, algo)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("oc", [ROW_MAJOR, COL_MAJOR])
def test_k_zero_sets_c_to_zero(dtype, oc):
    p = gi.make_problem(37, 45, 0, dtype, order_c=oc, pad_c=3)
    flat = run(p)
    C = logical_c(p, flat)
    assert np.all(C == 0) and padding_untouched(p, flat)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(0, 5, 7), (5, 0, 7), (0, 0, 0)])
def test_empty_output_untouched(dtype, shape):
    p = gi.make_problem(*shape, dtype)
    flat = run(p)
    assert np.all(np.isnan(flat))


# --- leading dimensions beyond the minimum, aligned and not -----------------------------
@pytest.mark.parametrize("dtype,algo", CASES, ids=CASE_IDS)
@pytest.mark.parametrize("pad", [1, 3, 8])
def test_padded_leading_dimensions(dtype, algo, pad):
    for orders in [(ROW_MAJOR, ROW_MAJOR, ROW_MAJOR), (ROW_MAJOR, COL_MAJOR, COL_MAJOR),
                   (COL_MAJOR, ROW_MAJOR, ROW_MAJOR)]:
        p = gi.make_problem(200, 264, 136, dtype, *orders, wid=43, pad_a=pad, pad_b=2 * pad,
                            pad_c=pad)
        check(p, algo)


# --- determinism: no atomics, so repeated runs agree bit for bit ------------------------
@pytest.mark.parametrize("dtype,algo", [("f32", g.Algo.REGBLOCK), ("f32", g.Algo.MFMA),
                                        ("bf16", g.Algo.MFMA_256x256), ("bf16", g.Algo.MFMA_128x128)],
                         ids=lambda x: str(x))
def test_repeated_runs_identical(dtype, algo):
    p = gi.make_problem(777, 1025, 513, dtype, ROW_MAJOR, COL_MAJOR, wid=44)
    A, B = to_device(p.A), to_device(p.B)
    first = run(p, algo, A, B)
    for _ in range(9):
        assert np.array_equal(run(p, algo, A, B), first, equal_nan=True)


# --- the torch-facing helper -------------------------------------------------------------
def test_matmul_helper_on_tensors_and_views():
    """The torch helper maps strides to (ld, order) for row- and column-major operands and C;
    references from the fp64 oracle on the same values."""
    import torch
    rng = np.random.default_rng(5)
    a32 = rng.uniform(-1, 1, (300, 200)).astype(np.float32)
    b32 = rng.uniform(-1, 1, (200, 100)).astype(np.float32)
    ref, D = oracle.gemm(300, 100, 200, a32.reshape(-1), 200, ROW_MAJOR, b32.reshape(-1), 100, ROW_MAJOR)
    a, b = torch.from_numpy(a32).cuda(), torch.from_numpy(b32).cuda()
    for x, y in [(a, b), (a.t().contiguous().t(), b), (a, b.t().contiguous().t())]:
        out = g.matmul(x, y)
        assert oracle.normalised_error(out.cpu().numpy(), ref, D) <= TOL["f32"]
    out_cm = torch.empty(100, 300, device="cuda").t()           # column-major C
    g.matmul(a, b, out=out_cm)
    assert oracle.normalised_error(out_cm.cpu().numpy(), ref, D) <= TOL["f32"]
    # 16-bit inputs: the oracle reads the same rounded values (bf16 bit patterns, fp16)
    ab, bb = a.bfloat16(), b.bfloat16()
    abits = ab.cpu().view(torch.int16).numpy().view(np.uint16).reshape(-1)
    bbits = bb.cpu().view(torch.int16).numpy().view(np.uint16).reshape(-1)
    refb, Db = oracle.gemm(300, 100, 200, abits, 200, ROW_MAJOR, bbits, 100, ROW_MAJOR)
    out = g.matmul(ab, bb.t().contiguous().t())
    assert oracle.normalised_error(out.cpu().numpy(), refb, Db) <= TOL["bf16"]
    assert g.gemm_last_kernel().startswith("bf16_")
    ah, bh = a.half(), b.half()
    refh, Dh = oracle.gemm(300, 100, 200, ah.cpu().numpy().reshape(-1), 200, ROW_MAJOR,
                           bh.cpu().numpy().reshape(-1), 100, ROW_MAJOR)
    out = g.matmul(ah, bh.t().contiguous().t())
    assert oracle.normalised_error(out.cpu().numpy(), refh, Dh) <= TOL["f16"]
    assert g.gemm_last_kernel().startswith("f16_")


# --- the small-problem kernel (row-major A; B column-major for BF16) ---------------------
SK_SHAPES = [(1, 1, 1), (5, 15, 7), (16, 16, 16), (17, 300, 100), (33, 64, 1000), (64, 257, 129),
             (16, 4096, 4096), (48, 33, 4095), (65, 40, 70), (256, 256, 256), (1000, 700, 1000),
             (129, 1025, 333), (4095, 1, 1023), (2000, 3, 64)]


@pytest.mark.parametrize("dtype,ob", [("bf16", COL_MAJOR), ("f32", COL_MAJOR), ("f32", ROW_MAJOR)],
                         ids=["bf16-RC", "f32-RC", "f32-RR"])
@pytest.mark.parametrize("shape", SK_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_skinny_random(dtype, ob, shape):
    M, N, K = shape
    p = gi.make_problem(M, N, K, dtype, ROW_MAJOR, ob, wid=50)
    check(p, g.Algo.SKINNY)
    assert g.gemm_last_kernel() == f"{dtype}_skinny16"


@pytest.mark.parametrize("dtype,ob", [("bf16", COL_MAJOR), ("f32", ROW_MAJOR)], ids=["bf16", "f32"])
@pytest.mark.parametrize("pad", [1, 3, 8])
def test_skinny_padded_and_misaligned(dtype, ob, pad):
    p = gi.make_problem(37, 130, 517, dtype, ROW_MAJOR, ob, wid=51, pad_a=pad, pad_b=pad, pad_c=pad)
    check(p, g.Algo.SKINNY)


@pytest.mark.parametrize("dtype,ob", [("bf16", COL_MAJOR), ("f32", ROW_MAJOR), ("f32", COL_MAJOR)],
                         ids=["bf16", "f32-RR", "f32-RC"])
def test_skinny_small_integer_exact(dtype, ob):
    rng = np.random.default_rng(9)
    M, N, K = 40, 200, 999
    A = rng.integers(-4, 5, (M, K)).astype(np.float32)
    B = rng.integers(-4, 5, (K, N)).astype(np.float32)
    check(gi.make_problem(M, N, K, dtype, ROW_MAJOR, ob, A_logical=A, B_logical=B),
          g.Algo.SKINNY, exact=True)


def test_skinny_column_major_c_uses_n_as_rows():
    # C column-major: the kernel computes C^T (N x M) = B^T A^T, so N <= 64 qualifies when B
    # is column-major (B^T row-major) and, for BF16, A row-major (A^T column-major)
    p = gi.make_problem(300, 20, 257, "bf16", ROW_MAJOR, COL_MAJOR, COL_MAJOR, wid=52)
    check(p, g.Algo.SKINNY)


# --- the small-problem kernel with four column blocks per workgroup (64 x 64 of C, K split
# over eight wavefronts): chosen when that still gives every CU a workgroup -------------------
SKINNY64_SHAPES = [(1000, 1000, 1000), (1030, 1000, 77), (1024, 1025, 1), (1001, 1023, 333), (1024, 1024, 4097)]


@pytest.mark.parametrize("dtype,ob", [("f32", ROW_MAJOR), ("f32", COL_MAJOR), ("bf16", COL_MAJOR)],
                         ids=["f32-RR", "f32-RC", "bf16"])
@pytest.mark.parametrize("shape", SKINNY64_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_skinny64_random(dtype, ob, shape):
    M, N, K = shape
    p = gi.make_problem(M, N, K, dtype, ROW_MAJOR, ob, wid=53)
    check(p, g.Algo.SKINNY, key=("skinny64", dtype, ob, shape))
    assert g.gemm_last_kernel() == f"{dtype}_skinny64"


@pytest.mark.parametrize("dtype,ob", [("f32", ROW_MAJOR), ("f32", COL_MAJOR), ("bf16", COL_MAJOR)],
                         ids=["f32-RR", "f32-RC", "bf16"])
def test_skinny64_small_integer_exact(dtype, ob):
    rng = np.random.default_rng(19)
    M, N, K = 1003, 1021, 301
    A = rng.integers(-4, 5, (M, K)).astype(np.float32)
    B = rng.integers(-4, 5, (K, N)).astype(np.float32)
    check(gi.make_problem(M, N, K, dtype, ROW_MAJOR, ob, A_logical=A, B_logical=B), g.Algo.SKINNY, exact=True)
    assert g.gemm_last_kernel() == f"{dtype}_skinny64"


@pytest.mark.parametrize("oc", [ROW_MAJOR, COL_MAJOR], ids=["C-row", "C-col"])
@pytest.mark.parametrize("pad", [1, 4])
def test_skinny64_padded_and_c_orders(oc, pad):
    # column-major C swaps the operands: B^T (column-major when B is row-major) becomes A
    ob = ROW_MAJOR if oc == ROW_MAJOR else COL_MAJOR
    p = gi.make_problem(1000, 1030, 260, "f32", ROW_MAJOR, ob, oc, wid=54, pad_a=pad, pad_b=pad, pad_c=pad)
    check(p, g.Algo.SKINNY)
    assert g.gemm_last_kernel() == "f32_skinny64"


@pytest.mark.parametrize("shape,pad", [((1000, 1004, 129), 3), ((1030, 1000, 300), 0), ((1000, 996, 4097), 5)],
                         ids=lambda v: str(v))
def test_skinny64_row_major_b_edge_slab_exact(shape, pad):
    """Row-major FP32 B with N % 4 == 0 and a last column slab that N ends inside: that slab takes
    the unchecked 16-byte loads, its lanes past N reading the slab's last valid columns.  Small
    integers make every element exact; the check also covers C's padding and, with padded rows of
    B, lanes that must not read past a row's N columns."""
    M, N, K = shape
    rng = np.random.default_rng(23)
    A = rng.integers(-4, 5, (M, K)).astype(np.float32)
    B = rng.integers(-4, 5, (K, N)).astype(np.float32)
    p = gi.make_problem(M, N, K, "f32", ROW_MAJOR, ROW_MAJOR, A_logical=A, B_logical=B, pad_b=pad, pad_c=pad)
    check(p, g.Algo.SKINNY, exact=True)
    assert g.gemm_last_kernel() == "f32_skinny64"


def test_skinny64_row_major_b_edge_slab_split_k():
    """The same edge slab with split-K through a workspace (partial tiles, then the slice sum)."""
    p = gi.make_problem(16, 1000, 16384, "f32", ROW_MAJOR, ROW_MAJOR, wid=66)
    flat, need, kernel = run_ws(p)
    assert need > 0 and kernel == "f32_skinny64_splitk"
    ref, D = oracle.gemm(p.M, p.N, p.K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b)
    assert oracle.normalised_error(logical_c(p, flat), ref, D) <= TOL["f32"]


@pytest.mark.parametrize("dtype,ob", [("f32", ROW_MAJOR), ("bf16", COL_MAJOR)], ids=["f32-RR", "bf16"])
def test_split_k_for_two_rounds_of_skinny_blocks(dtype, ob):
    """16 rows and 8192 columns: 512 blocks of 16 columns would take two rounds; with a workspace
    the call runs one round of 64-column blocks in K slices and sums the slices in order."""
    p = gi.make_problem(16, 8192, 2048, dtype, ROW_MAJOR, ob, wid=67)
    flat, need, kernel = run_ws(p)
    assert need > 0 and kernel == f"{dtype}_skinny64_splitk"
    ref, D = oracle.gemm(p.M, p.N, p.K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b)
    assert oracle.normalised_error(logical_c(p, flat), ref, D) <= TOL[dtype]
    again, _, _ = run_ws(p)
    assert np.array_equal(flat, again)         # fixed slice order: bit-identical repeats


# --- few FP32 rows with row-major B: 32-column blocks over two K halves, added into a zeroed C
HALVES_CASES = [((16, 4096, 4096), (ROW_MAJOR, ROW_MAJOR, ROW_MAJOR)),
                ((1, 4096, 4096), (ROW_MAJOR, ROW_MAJOR, ROW_MAJOR)),
                ((13, 4094, 4097), (ROW_MAJOR, ROW_MAJOR, ROW_MAJOR)),
                ((16, 2048, 8192), (ROW_MAJOR, ROW_MAJOR, ROW_MAJOR)),
                ((7, 3000, 6001), (ROW_MAJOR, ROW_MAJOR, ROW_MAJOR)),
                ((16, 2080, 4096), (ROW_MAJOR, ROW_MAJOR, ROW_MAJOR)),
                # column-major C: C^T = B^T A^T is the 16-row problem
                ((4096, 16, 4096), (COL_MAJOR, COL_MAJOR, COL_MAJOR))]


@pytest.mark.parametrize("shape,orders", HALVES_CASES, ids=lambda v: str(v))
def test_skinny_halves_random(shape, orders):
    """The default choice for few rows of an FP32 product with row-major A and B, a long K and
    an even N and ldb: a workgroup per 32-column block and K half, each adding its sum into C
    after C is zeroed; ragged N (the last block's lanes past N read the last valid column pair)
    and ragged K (the second half shorter) included."""
    M, N, K = shape
    p = gi.make_problem(M, N, K, "f32", *orders, wid=68)
    check(p, g.Algo.AUTO, key=("halves", shape, orders))
    assert g.gemm_last_kernel() == "f32_skinny32_halves"


def test_skinny_halves_small_integer_exact_and_repeatable():
    """Small integers: exact under any order, so bit-exact; padded B (even ldb) and a padded,
    misaligned C whose padding must stay untouched.  Random inputs: two calls give the same bits,
    since each output gets exactly two atomic contributions and 0 + x + y = 0 + y + x."""
    rng = np.random.default_rng(29)
    M, N, K = 16, 4090, 4097
    A = rng.integers(-4, 5, (M, K)).astype(np.float32)
    B = rng.integers(-4, 5, (K, N)).astype(np.float32)
    p = gi.make_problem(M, N, K, "f32", ROW_MAJOR, ROW_MAJOR, A_logical=A, B_logical=B, pad_b=2, pad_c=3)
    check(p, g.Algo.AUTO, exact=True)
    assert g.gemm_last_kernel() == "f32_skinny32_halves"
    q = gi.make_problem(16, 4096, 4096, "f32", ROW_MAJOR, ROW_MAJOR, wid=69)
    first, again = run(q, g.Algo.AUTO), run(q, g.Algo.AUTO)
    assert g.gemm_last_kernel() == "f32_skinny32_halves"
    assert np.array_equal(first.view(np.uint32), again.view(np.uint32))


@pytest.mark.parametrize("shape,pad_b,ob", [((16, 4095, 4096), 0, ROW_MAJOR), ((16, 4094, 4096), 1, ROW_MAJOR),
                                            ((16, 4096, 2048), 0, ROW_MAJOR), ((17, 4096, 4096), 0, ROW_MAJOR),
                                            ((16, 4096, 4096), 0, COL_MAJOR)], ids=lambda v: str(v))
def test_skinny_halves_not_taken(shape, pad_b, ob):
    """Odd N, odd ldb (column pairs not 8-byte aligned), K below the split's minimum, two 16-row
    strips, column-major B: 16-column blocks over the whole of K, as before."""
    M, N, K = shape
    p = gi.make_problem(M, N, K, "f32", ROW_MAJOR, ob, wid=70, pad_b=pad_b)
    check(p, g.Algo.AUTO, key=("halves-not", shape, pad_b, ob))
    assert g.gemm_last_kernel() == "f32_skinny16"


PAIRS_CASES = [((16, 8192, 4096), 0), ((1, 8192, 512), 0), ((13, 8190, 1025), 2), ((7, 9000, 5001), 0),
               ((16, 5120, 777), 4)]


@pytest.mark.parametrize("shape,pad", PAIRS_CASES, ids=lambda v: str(v))
def test_skinny_pairs_random(shape, pad):
    """Few FP32 rows whose 16-column blocks would take more than one round: 32-column blocks
    over the whole of K, plain stores; ragged N and K, padded (even) ldb and padded C."""
    M, N, K = shape
    p = gi.make_problem(M, N, K, "f32", ROW_MAJOR, ROW_MAJOR, wid=72, pad_b=pad, pad_c=pad + 1)
    check(p, g.Algo.AUTO, key=("pairs", shape, pad))
    assert g.gemm_last_kernel() == "f32_skinny32"


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", [(16, 8192, 1024), (9, 8191, 777), (16, 5123, 2049)], ids=lambda s: "x".join(map(str, s)))
def test_skinny_pairs_column_major_b(dtype, shape):
    """The same one round of 32-column blocks for a column-major B: two plain 16-column blocks per
    workgroup, any input type, odd N included (the last block's columns past N are clamped)."""
    M, N, K = shape
    p = gi.make_problem(M, N, K, dtype, ROW_MAJOR, COL_MAJOR, wid=73)
    check(p, g.Algo.AUTO, key=("pairs-c", dtype, shape))
    assert g.gemm_last_kernel() == f"{dtype}_skinny32"


def test_skinny_pairs_small_integer_exact():
    rng = np.random.default_rng(31)
    M, N, K = 16, 8194, 1500
    A = rng.integers(-4, 5, (M, K)).astype(np.float32)
    B = rng.integers(-4, 5, (K, N)).astype(np.float32)
    check(gi.make_problem(M, N, K, "f32", ROW_MAJOR, ROW_MAJOR, A_logical=A, B_logical=B), g.Algo.AUTO, exact=True)
    assert g.gemm_last_kernel() == "f32_skinny32"


def test_skinny_halves_through_the_workspace_call():
    """A workspace does not change the choice where the 16-column blocks make one exact round."""
    p = gi.make_problem(16, 4096, 4096, "f32", ROW_MAJOR, ROW_MAJOR, wid=71)
    flat, need, kernel = run_ws(p)
    assert need == 0 and kernel == "f32_skinny32_halves"
    ref, D = oracle.gemm(p.M, p.N, p.K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b)
    assert oracle.normalised_error(logical_c(p, flat), ref, D) <= TOL["f32"]


def test_skinny64_closed_forms():
    n = 1024
    perm = np.random.default_rng(11).permutation(n)
    P = np.eye(n, dtype=np.float32)[perm]
    B = np.random.default_rng(12).uniform(-1, 1, (n, n)).astype(np.float32)
    pb = gi.make_problem(n, n, n, "f32", ROW_MAJOR, ROW_MAJOR, A_logical=P, B_logical=B)
    assert np.array_equal(logical_c(pb, run(pb, g.Algo.SKINNY)), B[perm])
    pa = gi.make_problem(n, n, n, "f32", ROW_MAJOR, ROW_MAJOR, A_logical=B, B_logical=P.T.copy())
    assert np.array_equal(logical_c(pa, run(pa, g.Algo.SKINNY)), B[:, perm])
    assert g.gemm_last_kernel() == "f32_skinny64"


@pytest.mark.parametrize("bad", [dict(order_a=COL_MAJOR), dict(dtype="bf16", order_b=ROW_MAJOR)],
                         ids=lambda d: str(d))
def test_skinny_rejects_unsupported(bad):
    kw = dict(M=16, N=64, K=64, dtype="f32", order_a=ROW_MAJOR, order_b=COL_MAJOR)
    kw.update(bad)
    with pytest.raises(g.GemmError) as e:
        run(gi.make_problem(**kw), g.Algo.SKINNY)
    assert e.value.status == g.Status.ERR_INVALID_VALUE


@pytest.mark.parametrize("dtype,shape,kernel", [
    ("f32", (16, 4096, 4096), "f32_skinny32_halves"), ("bf16", (16, 4096, 4096), "bf16_skinny16"),
    ("f32", (256, 256, 256), "f32_skinny16"), ("f32", (1000, 1000, 1000), "f32_skinny64"),
    ("f32", (2048, 2048, 256), "f32_dma128x128"), ("f32", (2047, 2049, 255), "f32_dma128x128"),
    ("f32", (4095, 4097, 1023), "f32_dma256x256"), ("bf16", (4095, 4097, 1023), "bf16_dma256x256"),
    ("bf16", (1000, 1000, 1000), "bf16_skinny64"), ("bf16", (768, 768, 768), "bf16_mfma64x64"),
    ("bf16", (800, 1200, 1000), "bf16_mfma64x64"),
    ("f32", (1500, 1500, 512), "f32_mfma64x64"), ("f32", (4096, 4096, 64), "f32_dma256x256"),
    ("bf16", (4096, 4096, 64), "bf16_dma256x256"),
    ("bf16", (2048, 4096, 128), "bf16_dma256x128"), ("bf16", (2048, 11008, 128), "bf16_dma256x256")],
    ids=lambda v: str(v))
def test_auto_kernel_choice(dtype, shape, kernel):
    """AUTO: few rows or too few 64 x 64 tiles -> small-problem kernel (for 16-bit inputs with
    K <= 2048 whose 64 x 64 tiles fill at least half but not all of the CUs: those tiles), else
    block tiles; a
    tile kernel whose last tiles along an edge would start a second round stops at the last
    whole tile there and leaves the rest to a strip (4095 x 4097 on 256^2 tiles: 16 x 16
    tiles and a one-column strip)."""
    M, N, K = shape
    p = gi.make_problem(M, N, K, dtype, ROW_MAJOR, COL_MAJOR if dtype == "bf16" else ROW_MAJOR, wid=52)
    if M * N * K > 2**31:
        # parity at this size: test_workloads_gpu (sampled outputs, same AUTO launch)
        C = logical_c(p, run(p, g.Algo.AUTO))
        assert np.all(np.isfinite(C)), "every output written"
    else:
        check(p, g.Algo.AUTO)
    assert g.gemm_last_kernel() == kernel


# --- plans of several launches: a core of tiles and strips for the rest of C (one-round cut:
# 2048 x 11008 BF16 runs 8 x 32 tiles of 256^2 and a 2048 x 2816 strip; 3000^2 FP32 an
# overhanging 128^2 core and strips; 6144^2 BF16 a 256 x 128 core and a 256^2 strip) -------
@pytest.mark.parametrize("dtype,shape", [("bf16", (2048, 11008, 64)), ("f32", (3000, 3000, 96)),
                                         ("bf16", (6144, 6144, 64)), ("f32", (4095, 4097, 40)),
                                         ("bf16", (4095, 4097, 72))], ids=lambda v: str(v))
def test_auto_core_and_strips(dtype, shape):
    M, N, K = shape
    p = gi.make_problem(M, N, K, dtype, ROW_MAJOR, COL_MAJOR if dtype == "bf16" else ROW_MAJOR, wid=56)
    check(p, g.Algo.AUTO)


# --- FP32 direct-copy kernel (16x16x4 matrix instructions, operands copied into LDS as laid
# out in memory) --------------------------------------------------------------------------
# ragged shapes: the last tiles overhang M (row-major A) or N (column-major B), or the
# other edges leave strips for a separate GEMM; (129, 128, 32) and (130, 384, 100) leave
# wavefronts of the last tile without a single row of A (or B) to copy
DMA_SHAPES = [(128, 128, 32), (256, 384, 64), (200, 256, 96), (128, 132, 32), (132, 644, 1024),
              (384, 128, 4096), (252, 388, 160), (128, 128, 36), (260, 132, 1000), (256, 256, 60),
              (129, 128, 32), (130, 384, 100), (383, 129, 33)]


@pytest.mark.parametrize("orders", ORDERS3, ids=lambda o: "".join("RC"[x] for x in o))
@pytest.mark.parametrize("shape", DMA_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f32_dma_random(orders, shape):
    M, N, K = shape
    oa, ob, oc = orders
    p = gi.make_problem(M, N, K, "f32", oa, ob, oc, wid=53)
    check(p, g.Algo.MFMA_DMA, key=("dma", orders, shape))
    assert g.gemm_last_kernel().startswith("f32_dma")


DMA256_SHAPES = [(256, 256, 32), (512, 768, 96), (300, 516, 64), (256, 1028, 224), (772, 260, 32),
                 (256, 256, 44), (516, 260, 1000), (257, 256, 64), (256, 257, 64), (511, 300, 95)]


@pytest.mark.parametrize("orders", ORDERS3, ids=lambda o: "".join("RC"[x] for x in o))
@pytest.mark.parametrize("shape", DMA256_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f32_dma256_random(orders, shape):
    """256 x 256 tiles of eight wavefronts; ragged shapes overhang M or N where that operand
    is k-contiguous and leave strips elsewhere."""
    M, N, K = shape
    oa, ob, oc = orders
    p = gi.make_problem(M, N, K, "f32", oa, ob, oc, wid=54)
    check(p, g.Algo.MFMA_256x256, key=("dma256", orders, shape))
    assert g.gemm_last_kernel() == "f32_dma256x256"


def test_f32_dma256_small_integer_exact():
    rng = np.random.default_rng(12)
    M, N, K = 520, 516, 640
    A = rng.integers(-4, 5, (M, K)).astype(np.float32)
    B = rng.integers(-4, 5, (K, N)).astype(np.float32)
    check(gi.make_problem(M, N, K, "f32", ROW_MAJOR, ROW_MAJOR, A_logical=A, B_logical=B),
          g.Algo.MFMA_256x256, exact=True)


@pytest.mark.parametrize("ob", [ROW_MAJOR, COL_MAJOR], ids=["RR", "RC"])
def test_f32_dma_small_integer_exact(ob):
    rng = np.random.default_rng(11)
    M, N, K = 300, 256, 640
    A = rng.integers(-4, 5, (M, K)).astype(np.float32)
    B = rng.integers(-4, 5, (K, N)).astype(np.float32)
    check(gi.make_problem(M, N, K, "f32", ROW_MAJOR, ob, A_logical=A, B_logical=B), g.Algo.MFMA_DMA,
          exact=True)


def test_f32_dma_closed_forms():
    n = 256
    ones = gi.make_problem(n, n, n, "f32", ROW_MAJOR, ROW_MAJOR, A_logical=np.ones((n, n), np.float32),
                           B_logical=np.ones((n, n), np.float32))
    C = logical_c(ones, run(ones, g.Algo.MFMA_DMA))
    assert np.all(C == n)
    perm = np.random.default_rng(3).permutation(n)
    P = np.eye(n, dtype=np.float32)[perm]
    B = np.random.default_rng(4).uniform(-1, 1, (n, n)).astype(np.float32)
    pb = gi.make_problem(n, n, n, "f32", ROW_MAJOR, ROW_MAJOR, A_logical=P, B_logical=B)
    assert np.array_equal(logical_c(pb, run(pb, g.Algo.MFMA_DMA)), B[perm])
    pa = gi.make_problem(n, n, n, "f32", ROW_MAJOR, ROW_MAJOR, A_logical=B, B_logical=P.T.copy())
    assert np.array_equal(logical_c(pa, run(pa, g.Algo.MFMA_DMA)), B[:, perm])


@pytest.mark.parametrize("bad", [dict(K=28), dict(N=100), dict(M=127), dict(order_a=COL_MAJOR, K=16)],
                         ids=lambda d: str(d))
def test_f32_dma_rejects_unsupported(bad):
    kw = dict(M=256, N=256, K=64, dtype="f32", order_a=ROW_MAJOR, order_b=ROW_MAJOR)
    kw.update(bad)
    p = gi.make_problem(**kw)
    with pytest.raises(g.GemmError) as e:
        run(p, g.Algo.MFMA_DMA)
    assert e.value.status == g.Status.ERR_INVALID_VALUE


# --- BF16 direct-copy kernel (eight wavefronts, row-major A and column-major B) ----------
BDMA_SHAPES = [(256, 256, 64), (512, 384, 128), (300, 264, 192), (256, 128, 64), (776, 392, 64),
               (1024, 1024, 1024)]


@pytest.mark.parametrize("oc", [ROW_MAJOR, COL_MAJOR], ids=["RCR", "RCC"])
@pytest.mark.parametrize("shape", BDMA_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bf16_dma_random(oc, shape):
    M, N, K = shape
    if oc == COL_MAJOR and (N < 256 or M < 128):
        pytest.skip("after the column-major-C swap the shape is below the smallest tile")
    p = gi.make_problem(M, N, K, "bf16", ROW_MAJOR, COL_MAJOR, oc, wid=55)
    check(p, g.Algo.MFMA_DMA, key=("bdma", oc, shape))
    assert g.gemm_last_kernel().startswith("bf16_dma")


def test_bf16_dma_small_integer_exact():
    rng = np.random.default_rng(13)
    M, N, K = 520, 392, 640
    A = rng.integers(-4, 5, (M, K)).astype(np.float32)
    B = rng.integers(-4, 5, (K, N)).astype(np.float32)
    check(gi.make_problem(M, N, K, "bf16", ROW_MAJOR, COL_MAJOR, A_logical=A, B_logical=B),
          g.Algo.MFMA_DMA, exact=True)


def test_bf16_dma_closed_forms():
    n = 256
    perm = np.random.default_rng(5).permutation(n)
    P = np.eye(n, dtype=np.float32)[perm]
    B = gi.bf16_bits_to_f32(gi.f32_to_bf16_bits(np.random.default_rng(6).uniform(-1, 1, (n, n)).astype(np.float32)))
    pb = gi.make_problem(n, n, n, "bf16", ROW_MAJOR, COL_MAJOR, A_logical=P, B_logical=B)
    assert np.array_equal(logical_c(pb, run(pb, g.Algo.MFMA_DMA)), B[perm])
    pa = gi.make_problem(n, n, n, "bf16", ROW_MAJOR, COL_MAJOR, A_logical=B, B_logical=P.T.copy())
    assert np.array_equal(logical_c(pa, run(pa, g.Algo.MFMA_DMA)), B[:, perm])


# (row-major B is taken when N % 8 == 0)
@pytest.mark.parametrize("bad", [dict(order_b=ROW_MAJOR, N=260), dict(order_a=COL_MAJOR),
                                 dict(order_a=COL_MAJOR, order_b=ROW_MAJOR), dict(K=63)],
                         ids=lambda d: str(d))
def test_bf16_dma_rejects_unsupported(bad):
    kw = dict(M=256, N=256, K=128, dtype="bf16", order_a=ROW_MAJOR, order_b=COL_MAJOR)
    kw.update(bad)
    p = gi.make_problem(**kw)
    with pytest.raises(g.GemmError) as e:
        run(p, g.Algo.MFMA_DMA)
    assert e.value.status == g.Status.ERR_INVALID_VALUE


# --- BF16 direct-copy kernel on ragged shapes: partial edge tiles (rows past M or N read as
# zero through the buffer range, stores guarded), a K tail staged with bounds checks, K
# below one k-tile ---------------------------------------------------------------------------
BDMA_RAGGED = [(1, 1, 64), (255, 129, 71), (257, 385, 65), (300, 200, 1000), (513, 127, 100),
               (1000, 260, 1023), (260, 1001, 130), (4000, 4000, 100), (33, 300, 127)]


@pytest.mark.parametrize("oc", [ROW_MAJOR, COL_MAJOR], ids=["RCR", "RCC"])
@pytest.mark.parametrize("shape", BDMA_RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_bf16_dma_ragged(oc, shape):
    M, N, K = shape
    p = gi.make_problem(M, N, K, "bf16", ROW_MAJOR, COL_MAJOR, oc, wid=59)
    check(p, g.Algo.MFMA_DMA, key=("bdma_ragged", oc, shape))
    assert g.gemm_last_kernel().startswith("bf16_dma")


@pytest.mark.parametrize("shape", [(300, 257, 129), (257, 300, 1000), (4000, 4000, 100)],
                         ids=lambda s: "x".join(map(str, s)))
def test_bf16_dma_ragged_small_integer_exact(shape):
    M, N, K = shape
    rng = np.random.default_rng(M + 3 * N + K)
    A = rng.integers(-4, 5, (M, K)).astype(np.float32)
    B = rng.integers(-4, 5, (K, N)).astype(np.float32)
    check(gi.make_problem(M, N, K, "bf16", ROW_MAJOR, COL_MAJOR, A_logical=A, B_logical=B),
          g.Algo.MFMA_DMA, exact=True)
    assert g.gemm_last_kernel().startswith("bf16_dma")


@pytest.mark.parametrize("oc", [ROW_MAJOR, COL_MAJOR], ids=["RCR", "RCC"])
@pytest.mark.parametrize("pad", [1, 3, 8])
def test_bf16_dma_ragged_padded(oc, pad):
    """Odd and padded leading dimensions with partial tiles and a K tail; C padding intact."""
    p = gi.make_problem(300, 260, 100, "bf16", ROW_MAJOR, COL_MAJOR, oc, wid=60, pad_a=pad, pad_b=pad,
                        pad_c=pad)
    check(p, g.Algo.MFMA_DMA)
    assert g.gemm_last_kernel().startswith("bf16_dma")


def test_bf16_dma_ragged_closed_forms():
    M, N, K = 300, 260, 100
    P = np.eye(M, dtype=np.float32)[np.random.default_rng(8).permutation(M)]
    B = np.random.default_rng(9).uniform(-1, 1, (M, N)).astype(np.float32)
    pb = gi.make_problem(M, N, M, "bf16", ROW_MAJOR, COL_MAJOR, A_logical=P, B_logical=B)
    assert np.array_equal(logical_c(pb, run(pb, g.Algo.MFMA_DMA)), P @ pb.b_f32())
    ones = gi.make_problem(M, N, K, "bf16", ROW_MAJOR, COL_MAJOR, A_logical=np.ones((M, K)),
                           B_logical=np.ones((K, N)))
    assert np.all(logical_c(ones, run(ones, g.Algo.MFMA_DMA)) == K)


# --- direct copies from rows that are not 16-byte aligned (element alignment only) --------
@pytest.mark.parametrize("orders", ORDERS3, ids=lambda o: "".join("RC"[x] for x in o))
@pytest.mark.parametrize("pad", [1, 2, 3])
def test_f32_dma_unaligned_rows(orders, pad):
    oa, ob, oc = orders
    p = gi.make_problem(260, 388, 100, "f32", oa, ob, oc, wid=56, pad_a=pad, pad_b=pad, pad_c=pad)
    check(p, g.Algo.MFMA_DMA)
    assert g.gemm_last_kernel().startswith("f32_dma")
    p = gi.make_problem(512, 256, 64, "f32", oa, ob, oc, wid=57, pad_a=pad, pad_b=pad)
    check(p, g.Algo.MFMA_256x256)


@pytest.mark.parametrize("oc", [ROW_MAJOR, COL_MAJOR], ids=["RCR", "RCC"])
@pytest.mark.parametrize("pad", [1, 3, 7])
def test_bf16_direct_unaligned_rows(oc, pad):
    p = gi.make_problem(512, 384, 192, "bf16", ROW_MAJOR, COL_MAJOR, oc, wid=58, pad_a=pad, pad_b=pad, pad_c=pad)
    check(p, g.Algo.MFMA_DMA)
    assert g.gemm_last_kernel().startswith("bf16_dma")
    check(p, g.Algo.MFMA_256x256)      # the direct-copy kernel's 256 x 256 ring
    assert g.gemm_last_kernel() == "bf16_dma256x256"


# --- split-K across workgroups with a caller's workspace (gemm_*_ws) ----------------------
def run_ws(p, ws_bytes=None, misalign=0):
    """C (flat) after one gemm_*_ws call with a fresh workspace; (C, bytes needed, kernel)."""
    import torch
    A, B = to_device(p.A), to_device(p.B)
    C = torch.full((gi.c_buffer_size(p.M, p.N, p.ldc, p.order_c),), float("nan"), dtype=torch.float32,
                   device="cuda")
    need = g.gemm_workspace_size(p.dtype, p.M, p.N, p.K, p.order_a, p.order_b, p.order_c)
    nbytes = need if ws_bytes is None else ws_bytes
    ws = torch.full((nbytes // 4 + 64,), float("nan"), dtype=torch.float32, device="cuda")
    fn = {"f32": g.gemm_f32_ws, "bf16": g.gemm_bf16_f32acc_ws, "f16": g.gemm_f16_f32acc_ws}[p.dtype]
    print(f"[gpu] ws {p.dtype} M={p.M} N={p.N} K={p.K} orders=({p.order_a},{p.order_b},{p.order_c}) "
          f"ws={nbytes}/{need}", flush=True)
    fn(p.M, p.N, p.K, A.data_ptr(), p.lda, p.order_a, B.data_ptr(), p.ldb, p.order_b, C.data_ptr(), p.ldc,
       p.order_c, ws.data_ptr() + misalign, nbytes, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return C.cpu().numpy(), need, g.gemm_last_kernel()


# shapes whose own blocks leave CUs idle (few columns of C, long K), ragged in M, N and K
WS_CASES = [("f32", ROW_MAJOR, (16, 1024, 16384)), ("f32", COL_MAJOR, (16, 1024, 16384)),
            ("bf16", COL_MAJOR, (16, 1024, 16384)), ("f32", ROW_MAJOR, (5, 1000, 3001)),
            ("bf16", COL_MAJOR, (33, 1030, 5000)), ("f32", ROW_MAJOR, (64, 512, 8193)),
            ("f32", COL_MAJOR, (1, 250, 20000)), ("bf16", COL_MAJOR, (48, 70, 20000)),
            ("f32", ROW_MAJOR, (16, 256, 65536))]


@pytest.mark.parametrize("dtype,ob,shape", WS_CASES, ids=lambda v: str(v))
@pytest.mark.parametrize("oc", [ROW_MAJOR, COL_MAJOR], ids=["C-R", "C-C"])
def test_split_k_with_workspace(dtype, ob, shape, oc):
    """K split across workgroups: parity with the oracle, a workspace actually used, and the
    same bits on a second call (the slices are summed in a fixed order)."""
    M, N, K = shape
    if oc == COL_MAJOR:
        # the library computes C^T = B^T A^T (N x M): the few rows are C's few columns, its A
        # is B^T (row-major when B is column-major) and its B is A^T (order flipped)
        M, N = N, M
        p = gi.make_problem(M, N, K, dtype, 1 - ob, COL_MAJOR, oc, wid=57)
    else:
        p = gi.make_problem(M, N, K, dtype, ROW_MAJOR, ob, oc, wid=57)
    flat, need, kernel = run_ws(p)
    assert need > 0 and kernel.endswith("_splitk"), (need, kernel)
    assert padding_untouched(p, flat)
    ref, D = oracle.gemm(p.M, p.N, p.K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b)
    err = oracle.normalised_error(logical_c(p, flat), ref, D)
    assert err <= TOL[dtype], err
    again, _, _ = run_ws(p)
    assert np.array_equal(flat.view(np.uint32), again.view(np.uint32)), "not deterministic"


# --- split-K on the 16-bit direct-copy kernel's 256 x 256 tiles (few tiles, long K) --------
# (M, N, K, order of C): the default choice with a workspace splits each of these (5 to 8
# slices; K = 3000 and 4999 leave a ragged K tail in the last slice; ragged M and N overhang)
TILE_SPLIT_CASES = [(1000, 1025, 3000, ROW_MAJOR), (1500, 700, 4999, COL_MAJOR), (2048, 1024, 4096, ROW_MAJOR),
                    (4096, 512, 4096, ROW_MAJOR)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", TILE_SPLIT_CASES, ids=lambda c: "x".join(map(str, c)))
def test_tile_split_k_with_workspace(dtype, case):
    M, N, K, oc = case
    p = gi.make_problem(M, N, K, dtype, ROW_MAJOR, COL_MAJOR, oc, wid=64, pad_c=3)
    flat, need, kernel = run_ws(p)
    assert need > 0 and kernel == f"{dtype}_dma256x256_splitk", (need, kernel)
    assert padding_untouched(p, flat)
    ref, D = reference(p, key=("tilesplit", dtype, case))
    err = oracle.normalised_error(logical_c(p, flat), ref, D)
    assert err <= TOL[dtype], err
    again, _, _ = run_ws(p)
    assert np.array_equal(flat.view(np.uint32), again.view(np.uint32)), "not deterministic"


# FP32 split-K on whole 256 x 256 direct-copy tiles: (M, N, K, orders A, B, C); every
# instantiation of the operand orders, a ragged last slice (K = 8000: 7 slices of 1024 and one of
# 832), a column-major C
F32_TILE_SPLIT_CASES = [(4096, 512, 4096, ROW_MAJOR, ROW_MAJOR, ROW_MAJOR),
                        (4096, 512, 8000, COL_MAJOR, COL_MAJOR, ROW_MAJOR),
                        (512, 4096, 4096, ROW_MAJOR, COL_MAJOR, COL_MAJOR),
                        (2048, 2048, 4096, COL_MAJOR, ROW_MAJOR, ROW_MAJOR)]


@pytest.mark.parametrize("case", F32_TILE_SPLIT_CASES, ids=lambda c: "x".join(map(str, c)))
def test_f32_tile_split_k_with_workspace(case):
    M, N, K, oa, ob, oc = case
    p = gi.make_problem(M, N, K, "f32", oa, ob, oc, wid=67, pad_c=4)
    flat, need, kernel = run_ws(p)
    assert need > 0 and kernel == "f32_dma256x256_splitk", (need, kernel)
    assert padding_untouched(p, flat)
    ref, D = reference(p, key=("f32tilesplit", case))
    err = oracle.normalised_error(logical_c(p, flat), ref, D)
    assert err <= TOL["f32"], err
    again, _, _ = run_ws(p)
    assert np.array_equal(flat.view(np.uint32), again.view(np.uint32)), "not deterministic"


def test_f32_tile_split_k_small_integer_exact():
    rng = np.random.default_rng(68)
    M, N, K = 4096, 512, 8000
    A = rng.integers(-4, 5, (M, K)).astype(np.float32)
    B = rng.integers(-4, 5, (K, N)).astype(np.float32)
    p = gi.make_problem(M, N, K, "f32", ROW_MAJOR, ROW_MAJOR, A_logical=A, B_logical=B)
    flat, need, kernel = run_ws(p)
    assert kernel == "f32_dma256x256_splitk"
    ref, _ = oracle.gemm(p.M, p.N, p.K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b)
    assert np.array_equal(logical_c(p, flat).astype(np.float64), ref)


def test_tile_split_k_small_integer_exact_and_closed_forms():
    rng = np.random.default_rng(65)
    M, N, K = 1000, 1025, 3000
    A = rng.integers(-4, 5, (M, K)).astype(np.float32)
    B = rng.integers(-4, 5, (K, N)).astype(np.float32)
    p = gi.make_problem(M, N, K, "bf16", ROW_MAJOR, COL_MAJOR, A_logical=A, B_logical=B)
    flat, need, kernel = run_ws(p)
    assert kernel == "bf16_dma256x256_splitk"
    ref, _ = oracle.gemm(p.M, p.N, p.K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b)
    assert np.array_equal(logical_c(p, flat).astype(np.float64), ref)
    ones = gi.make_problem(M, N, K, "bf16", ROW_MAJOR, COL_MAJOR, A_logical=np.ones((M, K)),
                           B_logical=np.ones((K, N)))
    flat, _, kernel = run_ws(ones)
    assert kernel == "bf16_dma256x256_splitk" and np.all(logical_c(ones, flat) == K)


def test_tile_split_k_workspace_too_small_runs_unsplit():
    p = gi.make_problem(1000, 1025, 3000, "bf16", ROW_MAJOR, COL_MAJOR, wid=66)
    need = g.gemm_workspace_size("bf16", p.M, p.N, p.K, p.order_a, p.order_b, p.order_c)
    flat, _, kernel = run_ws(p, ws_bytes=need - 16)
    assert not kernel.endswith("_splitk"), kernel
    ref, D = reference(p, key=("tilesplit-small", 1))
    assert oracle.normalised_error(logical_c(p, flat), ref, D) <= TOL["bf16"]


def test_split_k_small_integer_exact():
    rng = np.random.default_rng(21)
    M, N, K = 16, 1024, 6000
    A = rng.integers(-3, 4, (M, K)).astype(np.float32)
    B = rng.integers(-3, 4, (K, N)).astype(np.float32)
    for dtype, ob in (("f32", ROW_MAJOR), ("bf16", COL_MAJOR)):
        p = gi.make_problem(M, N, K, dtype, ROW_MAJOR, ob, A_logical=A, B_logical=B)
        flat, need, kernel = run_ws(p)
        assert need > 0 and kernel.endswith("_splitk")
        ref, _ = oracle.gemm(p.M, p.N, p.K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b)
        assert np.array_equal(logical_c(p, flat).astype(np.float64), ref)


@pytest.mark.parametrize("dtype,ob", [("f32", ROW_MAJOR), ("bf16", COL_MAJOR)], ids=["f32", "bf16"])
def test_workspace_too_small_or_absent_runs_the_plain_path(dtype, ob):
    p = gi.make_problem(16, 1024, 16384, dtype, ROW_MAJOR, ob, wid=58)
    plain = run(p)
    plain_kernel = g.gemm_last_kernel()
    need = g.gemm_workspace_size(dtype, p.M, p.N, p.K, p.order_a, p.order_b, p.order_c)
    assert need > 0
    for nbytes in (0, need - 4):
        flat, _, kernel = run_ws(p, ws_bytes=nbytes)
        assert kernel == plain_kernel
        assert np.array_equal(flat.view(np.uint32), plain.view(np.uint32))


def test_workspace_must_be_16_byte_aligned():
    p = gi.make_problem(16, 4096, 4096, "f32", ROW_MAJOR, ROW_MAJOR, wid=59)
    with pytest.raises(g.GemmError) as e:
        run_ws(p, misalign=4)
    assert e.value.status == g.Status.ERR_INVALID_VALUE


# --- FP16 inputs (the same 16-bit kernels with the fp16 matrix instructions) --------------
F16_AUTO = [((4096, 4096, 256), "f16_dma256x256"), ((2048, 4096, 128), "f16_dma256x128"),
            ((1000, 1000, 1000), "f16_skinny64"), ((768, 768, 768), "f16_mfma64x64"),
            ((16, 4096, 4096), "f16_skinny16"),
            ((4095, 4097, 72), "f16_dma256x256"), ((300, 264, 192), None), ((33, 300, 127), None)]


@pytest.mark.parametrize("shape,kernel", F16_AUTO, ids=lambda v: str(v))
@pytest.mark.parametrize("oc", [ROW_MAJOR, COL_MAJOR], ids=["RCR", "RCC"])
def test_f16_auto(shape, kernel, oc):
    M, N, K = shape
    if oc == COL_MAJOR:
        kernel = None                      # C^T is another problem; parity only
    p = gi.make_problem(M, N, K, "f16", ROW_MAJOR, COL_MAJOR, oc, wid=60)
    check(p, g.Algo.AUTO, key=("f16auto", shape, oc))
    if kernel:
        assert g.gemm_last_kernel() == kernel


F16_FORCED = [(g.Algo.MFMA_DMA, (257, 385, 65)), (g.Algo.MFMA_DMA, (512, 384, 200)),
              (g.Algo.MFMA_256x256, (300, 516, 96)), (g.Algo.MFMA_256x128, (260, 200, 70)),
              (g.Algo.MFMA_128x128, (129, 257, 33)), (g.Algo.MFMA_64x64, (65, 100, 130)),
              (g.Algo.SKINNY, (40, 700, 999))]


@pytest.mark.parametrize("algo,shape", F16_FORCED, ids=lambda v: str(v))
def test_f16_forced_kernels(algo, shape):
    M, N, K = shape
    p = gi.make_problem(M, N, K, "f16", ROW_MAJOR, COL_MAJOR, wid=61)
    check(p, algo)
    assert g.gemm_last_kernel().startswith("f16_")


@pytest.mark.parametrize("orders", [(ROW_MAJOR, ROW_MAJOR), (COL_MAJOR, COL_MAJOR), (COL_MAJOR, ROW_MAJOR)],
                         ids=["RR", "CC", "CR"])
def test_f16_other_layouts(orders):
    """Operands that are not both k-contiguous take the register-staged 16-bit kernel."""
    oa, ob = orders
    p = gi.make_problem(200, 300, 150, "f16", oa, ob, wid=62, pad_a=3, pad_b=1)
    check(p, g.Algo.AUTO)
    assert g.gemm_last_kernel().startswith("f16_mfma")


def test_f16_small_integer_exact():
    rng = np.random.default_rng(31)
    M, N, K = 520, 392, 640
    A = rng.integers(-8, 9, (M, K)).astype(np.float32)
    B = rng.integers(-8, 9, (K, N)).astype(np.float32)
    check(gi.make_problem(M, N, K, "f16", ROW_MAJOR, COL_MAJOR, A_logical=A, B_logical=B), g.Algo.AUTO,
          exact=True)


@pytest.mark.parametrize("algo,shape", [(g.Algo.AUTO, (256, 256, 1024)), (g.Algo.AUTO, (16, 512, 2048)),
                                        (g.Algo.AUTO, (2048, 2048, 256)), (g.Algo.MFMA_DMA, (512, 512, 256)),
                                        (g.Algo.MFMA_256x256, (256, 256, 128))], ids=str)
def test_f16_values_bf16_cannot_hold(algo, shape):
    """1 + 2^-10 is exact in fp16 and not in bf16 (7 fraction bits): a kernel that read the
    fp16 patterns as bf16 would be far off.  Also a subnormal (2^-20) and a value near the
    top of the fp16 range (61440 = 15 * 2^12), products exact in FP32."""
    M, N, K = shape
    A = np.full((M, K), 1.0 + 2.0 ** -10, np.float32)
    A[:, 1] = 2.0 ** -20
    A[:, 2] = 61440.0
    B = np.ones((K, N), np.float32)
    p = gi.make_problem(M, N, K, "f16", ROW_MAJOR, COL_MAJOR, A_logical=A, B_logical=B)
    C = logical_c(p, run(p, algo))
    want = (K - 2) * (1.0 + 2.0 ** -10) + 2.0 ** -20 + 61440.0
    ref, D = oracle.gemm(p.M, p.N, p.K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b)
    assert ref[0, 0] == want
    assert oracle.normalised_error(C, ref, D) <= TOL["f16"]


def test_f16_rejects_the_vector_ladder():
    p = gi.make_problem(256, 256, 64, "f16", ROW_MAJOR, COL_MAJOR)
    for algo in (g.Algo.NAIVE, g.Algo.REGBLOCK):
        with pytest.raises(g.GemmError) as e:
            run(p, algo)
        assert e.value.status == g.Status.ERR_INVALID_VALUE


def test_f16_split_k_with_workspace():
    p = gi.make_problem(16, 1024, 16384, "f16", ROW_MAJOR, COL_MAJOR, wid=63)
    flat, need, kernel = run_ws(p)
    assert need > 0 and kernel == "f16_skinny64_splitk"
    ref, D = oracle.gemm(p.M, p.N, p.K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b)
    assert oracle.normalised_error(logical_c(p, flat), ref, D) <= TOL["f16"]
