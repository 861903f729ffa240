"""GPU parity of the 16-bit direct-copy kernel on row-major B (n contiguous: PyTorch's `a @ b`
layout, attention's P.V) against the fp64 oracle.

That build keeps B's k-tile in LDS as it lies in memory and reads it with the transposing LDS
read; it takes row-major A with row-major B (after the column-major-C swap: also all three
column-major) when N % 8 == 0 and K >= 64.  The bar is the 16-bit one: normalised error <= 1e-4
for random values, bit for bit where every summation order is exact (small integers,
permutations, ones).
"""
import numpy as np
import pytest

import gemm_f32_amd as g
import gemm_inputs as gi
import oracle
from gemm_inputs import COL_MAJOR, ROW_MAJOR
from gpu_util import TOL, check, check_batched, logical_c, run, to_device

pytestmark = pytest.mark.gpu

R, C_ = ROW_MAJOR, COL_MAJOR

# whole tiles; several tiles with a K tail; ragged M with N a multiple of 8 but not of the tile;
# one k-tile; K one past a k-tile; a single column chunk (N = 8); one output row
SHAPES = [(512, 512, 256), (1000, 264, 1023), (257, 392, 65), (300, 136, 64), (33, 520, 200),
          (520, 8, 640), (1, 4096, 128), (768, 1288, 2048), (4095, 4104, 96)]


# both tile configurations of the direct-copy kernel, chosen explicitly (the default choice
# gives small problems to other kernels)
TILES = {g.Algo.MFMA_256x256: "dma256x256", g.Algo.MFMA_256x128: "dma256x128"}
TILE_IDS = ["256x256", "256x128"]


@pytest.mark.parametrize("algo", list(TILES), ids=TILE_IDS)
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_row_major_b_random(dtype, shape, algo):
    M, N, K = shape
    p = gi.make_problem(M, N, K, dtype, R, R, R, wid=80)
    check(p, algo, key=("brm", dtype, shape))
    assert g.gemm_last_kernel() == f"{dtype}_{TILES[algo]}"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("orders", [(C_, C_, C_), (R, R, C_)], ids=["CCC", "RRC"])
def test_other_orders_reaching_row_major_b(dtype, orders):
    """All column-major becomes row-major A and B after the swap (the kernel runs on C^T); R,R,C
    becomes column-major A and B (another kernel).  Both against the oracle."""
    p = gi.make_problem(600, 392, 333, dtype, *orders, wid=81)
    if orders == (C_, C_, C_):
        check(p, g.Algo.MFMA_256x256)
        assert g.gemm_last_kernel() == f"{dtype}_dma256x256"
    else:
        check(p)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape,kernel", [((4096, 4096, 512), "dma256x256"), ((300, 260, 128), None)], ids=str)
def test_row_major_b_kernel_choice(dtype, shape, kernel):
    """The default choice: row-major B with N % 8 == 0 takes the direct-copy tiles where they
    fill the chip; N % 8 != 0 (260) the register-staged ones."""
    p = gi.make_problem(*shape, dtype, R, R, R, wid=82)
    check(p)
    name = g.gemm_last_kernel()
    assert name == f"{dtype}_{kernel}" if kernel else "_mfma" in name


@pytest.mark.parametrize("algo", list(TILES), ids=TILE_IDS)
@pytest.mark.parametrize("pad_b", [1, 3, 8, 120])
def test_row_major_b_padded_rows(pad_b, algo):
    """Leading dimensions beyond N, odd ones putting rows at 2-byte-aligned addresses; the
    padding holds NaN, so reading it for a stored column poisons C."""
    p = gi.make_problem(700, 392, 300, "bf16", R, R, R, wid=83, pad_a=5, pad_b=pad_b, pad_c=7)
    check(p, algo)
    assert g.gemm_last_kernel() == f"bf16_{TILES[algo]}"


@pytest.mark.parametrize("algo", list(TILES), ids=TILE_IDS)
@pytest.mark.parametrize("K", [64, 65, 71, 127, 128, 129, 191, 200, 1000])
def test_row_major_b_k_tails(K, algo):
    p = gi.make_problem(520, 392, K, "bf16", R, R, R, wid=84)
    check(p, algo)
    assert g.gemm_last_kernel() == f"bf16_{TILES[algo]}"


@pytest.mark.parametrize("algo", list(TILES), ids=TILE_IDS)
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(520, 392, 640), (300, 264, 129), (4096, 2048, 256)],
                         ids=lambda s: "x".join(map(str, s)))
def test_row_major_b_small_integer_exact(dtype, shape, algo):
    """Integers in [-4, 4]: every product and partial sum is exact in FP32."""
    M, N, K = shape
    rng = np.random.default_rng(M + 3 * N + K)
    A = rng.integers(-4, 5, (M, K)).astype(np.float32)
    B = rng.integers(-4, 5, (K, N)).astype(np.float32)
    p = gi.make_problem(M, N, K, dtype, R, R, R, A_logical=A, B_logical=B)
    check(p, algo, exact=True)


@pytest.mark.parametrize("algo", list(TILES), ids=TILE_IDS)
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_row_major_b_closed_forms(dtype, algo):
    """A = permutation gives B's rows and B = permutation gives A's columns, bit for bit; ones
    give K.  A transposed B tile, a wrong column of the transposing read or a k paired with
    the wrong A column fails these."""
    n = 520
    perm = np.random.default_rng(9).permutation(n)
    P = np.eye(n, dtype=np.float32)[perm]
    Rm = np.random.default_rng(10).uniform(-1, 1, (n, n)).astype(np.float32)
    pb = gi.make_problem(n, n, n, dtype, R, R, R, A_logical=P, B_logical=Rm)
    assert np.array_equal(logical_c(pb, run(pb, algo)), pb.b_f32()[perm])
    pa = gi.make_problem(n, n, n, dtype, R, R, R, A_logical=Rm, B_logical=P.T.copy())
    assert np.array_equal(logical_c(pa, run(pa, algo)), pa.a_f32()[:, perm])
    K = 1000
    ones = gi.make_problem(300, 264, K, dtype, R, R, R, A_logical=np.ones((300, K)), B_logical=np.ones((K, 264)))
    assert np.all(logical_c(ones, run(ones, algo)) == K)
    assert g.gemm_last_kernel() == f"{dtype}_{TILES[algo]}"


@pytest.mark.parametrize("algo", list(TILES), ids=TILE_IDS)
def test_row_major_b_each_element_of_b_in_place(algo):
    """B with a single nonzero per k-row (row k holds k+1 at column (37 k) mod N) and A = I: C
    is B, so each B element must land at its own row and column."""
    n, N = 512, 392
    B = np.zeros((n, N), np.float32)
    B[np.arange(n), (37 * np.arange(n)) % N] = np.arange(1, n + 1)
    p = gi.make_problem(n, N, n, "bf16", R, R, R, A_logical=np.eye(n, dtype=np.float32), B_logical=B)
    assert np.array_equal(logical_c(p, run(p, algo)), p.b_f32())


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_row_major_b_batched_small(dtype):
    """Four entries of row-major (2048 x 2048) . (2048 x 128), every entry against the oracle."""
    p = gi.make_batched_problem(4, 2048, 128, 2048, dtype, R, R, R, wid=85)
    check_batched(p)


def test_row_major_b_attention_pv_workload():
    """Attention's P.V at full size (32 heads, V rows 4096 apart): the direct-copy tiles run it;
    sampled outputs of four entries against the oracle."""
    from gpu_util import run_batched
    p = gi.workload_problem("attn_pv_32x2048x128x2048_bf16")
    got = p.c_view(run_batched(p))
    assert g.gemm_last_kernel().startswith("bf16_dma")
    for z in (0, 1, 17, 31):
        rng = np.random.default_rng(z)
        rows, cols = rng.integers(0, p.M, 1024), rng.integers(0, p.N, 1024)
        ref, D = oracle.gemm_sampled(p.M, p.N, p.K, p.A[z * p.sa:], p.lda, p.order_a, p.B[z * p.sb:], p.ldb,
                                     p.order_b, rows, cols)
        assert oracle.normalised_error(got[z][rows, cols], ref, D) <= TOL["bf16"]


def test_row_major_b_batched_strides_and_broadcast():
    """Padded leading dimensions, gaps between entries and one B for every entry (stride 0)."""
    p = gi.make_batched_problem(3, 300, 264, 200, "bf16", R, R, R, lda=205, ldb=270, sb=0, ldc=300, wid=86)
    check_batched(p)


def test_row_major_b_split_k_workspace():
    """A split-K plan on row-major B (4096 x 512 x 4096 with workspace): every slice against the
    oracle through the sum of slabs."""
    import torch
    M, N, K = 4096, 512, 4096
    p = gi.make_problem(M, N, K, "bf16", R, R, R, wid=87)
    ws_bytes = g.gemm_workspace_size("bf16", M, N, K, R, R, R)
    assert ws_bytes > 0
    A, B = to_device(p.A), to_device(p.B)
    C = torch.full((M * N,), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device="cuda")
    print(f"[gpu] split-K row-major B {M}x{N}x{K}", flush=True)
    g.gemm_bf16_f32acc_ws(M, N, K, A.data_ptr(), p.lda, R, B.data_ptr(), p.ldb, R, C.data_ptr(), p.ldc, R,
                          ws.data_ptr(), ws_bytes, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert g.gemm_last_kernel() == "bf16_dma256x256_splitk"
    rng = np.random.default_rng(12)
    rows, cols = rng.integers(0, M, 2048), rng.integers(0, N, 2048)
    ref, D = oracle.gemm_sampled(M, N, K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b, rows, cols)
    got = C.cpu().numpy().reshape(M, N)[rows, cols]
    assert oracle.normalised_error(got, ref, D) <= TOL["bf16"]


def test_row_major_b_square4096_sampled():
    """The 4096^3 problem on row-major B: 2048 sampled outputs against the oracle."""
    n = 4096
    p = gi.make_problem(n, n, n, "bf16", R, R, R, wid=3)
    C = logical_c(p, run(p))
    assert g.gemm_last_kernel() == "bf16_dma256x256"
    rng = np.random.default_rng(13)
    rows, cols = rng.integers(0, n, 2048), rng.integers(0, n, 2048)
    ref, D = oracle.gemm_sampled(n, n, n, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b, rows, cols)
    assert oracle.normalised_error(C[rows, cols], ref, D) <= TOL["bf16"]
