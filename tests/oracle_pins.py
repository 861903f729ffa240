"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each pin takes a loaded oracle library handle and raises AssertionError when the
oracle disagrees with:
  * exact rational arithmetic on tiny shapes (brute force with fractions.Fraction);
  * numpy's float64 matmul on the logical matrices (a library routine the oracle does
    not call);
  * closed forms: all-ones operands give C = K; an all-ones A gives column sums of B;
    identity and permutation operands reproduce / permute the other operand exactly;
  * small-integer operands, whose product is exact under any summation order;
  * invariants: (A.B)^T = B^T.A^T, and splitting K into two ranges and adding the
    partial products gives the full product -- the 4 x 4, tile-2 worked example of
    "GEMM" (Part 4 of How to make your models fast), section "A small example";
  * the multiply-add count M*N*K (FLOPs = 2MNK: "How a Matrix Multiply Runs on a GPU",
    section "The problem and the roofline"; "A06 - Tiled Matrix Multiply (GEMM)",
    section "The derivation that explains everything").

The same pins run against deliberately broken builds of the oracle (see
test_oracle_mutants.py) to show that each plausible mistake fails at least one.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import gemm_inputs as gi
import oracle
from gemm_inputs import COL_MAJOR, ROW_MAJOR

ORDERS = [(oa, ob) for oa in (ROW_MAJOR, COL_MAJOR) for ob in (ROW_MAJOR, COL_MAJOR)]
# every input type of the one-problem oracle: fp32, bf16, fp16 and the 8-bit formats (also mixed)
DTYPES = ("f32", "bf16", "f16", "e4m3", "e5m2", "e4m3_e5m2")
BATCH_DTYPES = ("f32", "bf16", "f16")


def _run(lib, p: gi.Problem, macs=False):
    return oracle.gemm(p.M, p.N, p.K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b,
                       lib=lib, return_macs=macs, **gi.oracle_formats(p))


def _int_matrix(rng, r, c, lo=-4, hi=4):
    return rng.integers(lo, hi + 1, size=(r, c)).astype(np.float32)


# ---------------------------------------------------------------------------------
def pin_fraction_bruteforce(lib):
    """Exact rational sums on tiny shapes: |C - exact| <= (K-1) * 2^-53 * D."""
    shapes = [(1, 1, 1), (2, 3, 4), (3, 1, 5), (4, 4, 4), (5, 7, 3), (8, 8, 8), (1, 6, 8)]
    for dtype in DTYPES:
        for (M, N, K) in shapes:
            for oa, ob in ORDERS:
                p = gi.make_problem(M, N, K, dtype, oa, ob, wid=101, pad_a=1, pad_b=2)
                C, D = _run(lib, p)
                a, b = p.a_f32(), p.b_f32()
                for i in range(M):
                    for j in range(N):
                        exact = sum((Fraction(float(a[i, k])) * Fraction(float(b[k, j]))
                                     for k in range(K)), Fraction(0))
                        dabs = sum((abs(Fraction(float(a[i, k])) * Fraction(float(b[k, j])))
                                    for k in range(K)), Fraction(0))
                        err = abs(Fraction(C[i, j]) - exact)
                        bound = Fraction(max(K - 1, 0)) * Fraction(2) ** -53 * dabs
                        assert err <= bound, (dtype, M, N, K, oa, ob, i, j)
                        assert abs(Fraction(D[i, j]) - dabs) <= bound, ("D", dtype, M, N, K, i, j)


def pin_numpy_crosscheck(lib):
    """numpy float64 matmul of the logical operands agrees to 1e-12 of D."""
    for dtype in DTYPES:
        for (M, N, K) in [(37, 53, 129), (64, 32, 16), (3, 100, 257)]:
            for oa, ob in ORDERS:
                p = gi.make_problem(M, N, K, dtype, oa, ob, wid=102, pad_a=3, pad_b=1)
                C, D = _run(lib, p)
                a = p.a_f32().astype(np.float64)
                b = p.b_f32().astype(np.float64)
                ref = a @ b
                dref = np.abs(a) @ np.abs(b)
                assert oracle.normalised_error(C, ref, dref) <= 1e-12, (dtype, M, N, K, oa, ob)
                assert np.max(np.abs(D - dref) / np.maximum(dref, 1e-300)) <= 1e-12


def pin_ones(lib):
    """A = ones, B = ones  =>  C == K exactly (16^3 is the pages' worked size)."""
    for (M, N, K) in [(16, 16, 16), (32, 32, 32), (64, 64, 64), (37, 45, 67)]:
        for dtype in DTYPES:
            for oa, ob in ORDERS:
                p = gi.make_problem(M, N, K, dtype, oa, ob, A_logical=np.ones((M, K)),
                                    B_logical=np.ones((K, N)))
                C, D = _run(lib, p)
                assert np.all(C == K) and np.all(D == K), (M, N, K, dtype, oa, ob)


def pin_ones_column_sums(lib):
    """A = ones  =>  C[i][j] = sum_k B[k][j] (integer-valued B: exact)."""
    rng = np.random.default_rng(7)
    for (M, N, K) in [(16, 16, 16), (5, 9, 33)]:
        Bl = _int_matrix(rng, K, N)
        colsum = Bl.astype(np.int64).sum(axis=0)
        for oa, ob in ORDERS:
            p = gi.make_problem(M, N, K, "f32", oa, ob, A_logical=np.ones((M, K)), B_logical=Bl)
            C, _ = _run(lib, p)
            assert np.array_equal(C, np.broadcast_to(colsum, (M, N)).astype(np.float64))


def pin_identity(lib):
    """A = I  =>  C == B bit for bit; B = I  =>  C == A bit for bit."""
    for n, other in [(16, 16), (32, 19), (7, 40)]:
        for dtype in DTYPES:
            for oa, ob in ORDERS:
                p = gi.make_problem(n, other, n, dtype, oa, ob, wid=103, A_logical=np.eye(n))
                C, _ = _run(lib, p)
                assert np.array_equal(C, p.b_f32().astype(np.float64)), ("A=I", n, dtype, oa, ob)
                q = gi.make_problem(other, n, n, dtype, oa, ob, wid=104, B_logical=np.eye(n))
                C, _ = _run(lib, q)
                assert np.array_equal(C, q.a_f32().astype(np.float64)), ("B=I", n, dtype, oa, ob)


def pin_permutation(lib):
    """A = P (permutation)  =>  rows of B permuted; B = P  =>  columns of A permuted."""
    rng = np.random.default_rng(11)
    for n, other in [(16, 16), (33, 20)]:
        perm = rng.permutation(n)
        P = np.zeros((n, n))
        P[np.arange(n), perm] = 1.0           # (P.X)[i] = X[perm[i]]
        for dtype in DTYPES:
            for oa, ob in ORDERS:
                p = gi.make_problem(n, other, n, dtype, oa, ob, wid=105, A_logical=P)
                C, _ = _run(lib, p)
                assert np.array_equal(C, p.b_f32()[perm].astype(np.float64)), ("A=P", dtype, oa, ob)
                q = gi.make_problem(other, n, n, dtype, oa, ob, wid=106, B_logical=P)
                C, _ = _run(lib, q)
                inv = np.argsort(perm)                # (X.P)[:, j] = X[:, inv[j]]
                assert np.array_equal(C, q.a_f32()[:, inv].astype(np.float64)), ("B=P", dtype, oa, ob)


def pin_small_integers(lib):
    """Entries in {-4..4}: every partial sum is an exact integer, so C is the integer product."""
    rng = np.random.default_rng(13)
    for (M, N, K) in [(16, 16, 16), (33, 17, 65), (1, 40, 7), (50, 1, 3)]:
        Al, Bl = _int_matrix(rng, M, K), _int_matrix(rng, K, N)
        exact = (Al.astype(np.int64) @ Bl.astype(np.int64)).astype(np.float64)
        dexact = (np.abs(Al).astype(np.int64) @ np.abs(Bl).astype(np.int64)).astype(np.float64)
        for dtype in DTYPES:
            for oa, ob in ORDERS:
                p = gi.make_problem(M, N, K, dtype, oa, ob, A_logical=Al, B_logical=Bl, pad_a=2)
                C, D = _run(lib, p)
                assert np.array_equal(C, exact), (M, N, K, dtype, oa, ob)
                assert np.array_equal(D, dexact), (M, N, K, dtype, oa, ob)


def pin_transpose(lib):
    """(A.B)^T computed as B^T.A^T from the same buffers (order flags flipped) agrees bitwise."""
    for dtype in DTYPES:
        for oa, ob in ORDERS:
            p = gi.make_problem(23, 31, 41, dtype, oa, ob, wid=107, pad_b=5)
            C, D = _run(lib, p)
            fm = gi.oracle_formats(p)
            Ct, Dt = oracle.gemm(p.N, p.M, p.K, p.B, p.ldb, 1 - p.order_b, p.A, p.lda,
                                 1 - p.order_a, lib=lib, fmt_a=fm.get("fmt_b"), fmt_b=fm.get("fmt_a"))
            assert np.array_equal(Ct, C.T) and np.array_equal(Dt, D.T), (dtype, oa, ob)


def pin_k_split(lib):
    """Split K at k0: C = A[:, :k0].B[:k0, :] + A[:, k0:].B[k0:, :].

    The 4 x 4 case with tile 2 is the pages' worked example of a block walking along K;
    small-integer entries make the identity exact.
    """
    rng = np.random.default_rng(17)
    for (M, N, K, k0) in [(4, 4, 4, 2), (8, 5, 13, 6), (16, 16, 16, 4)]:
        Al, Bl = _int_matrix(rng, M, K), _int_matrix(rng, K, N)
        full, _ = _run(lib, gi.make_problem(M, N, K, "f32", A_logical=Al, B_logical=Bl))
        lo, _ = _run(lib, gi.make_problem(M, N, k0, "f32", A_logical=Al[:, :k0], B_logical=Bl[:k0]))
        hi, _ = _run(lib, gi.make_problem(M, N, K - k0, "f32", A_logical=Al[:, k0:], B_logical=Bl[k0:]))
        assert np.array_equal(full, lo + hi), (M, N, K, k0)
    # the worked example written out for C00 of the 4 x 4 case
    Al, Bl = _int_matrix(rng, 4, 4), _int_matrix(rng, 4, 4)
    C, _ = _run(lib, gi.make_problem(4, 4, 4, "f32", A_logical=Al, B_logical=Bl))
    c00 = Al[0, 0] * Bl[0, 0] + Al[0, 1] * Bl[1, 0] + Al[0, 2] * Bl[2, 0] + Al[0, 3] * Bl[3, 0]
    assert C[0, 0] == c00


def pin_mac_count(lib):
    """The loop nest performs exactly M*N*K multiply-adds."""
    for (M, N, K) in [(1, 1, 1), (3, 5, 7), (16, 16, 16), (0, 4, 4), (4, 0, 4), (4, 4, 0)]:
        p = gi.make_problem(M, N, K, "f32", wid=108)
        C, D, macs = _run(lib, p, macs=True)
        assert macs == M * N * K, (M, N, K, macs)


def pin_degenerate(lib):
    """K = 0 gives the empty sum C = 0; M or N = 0 gives an empty C."""
    p = gi.make_problem(5, 6, 0, "f32")
    C, D = _run(lib, p)
    assert C.shape == (5, 6) and np.all(C == 0) and np.all(D == 0)
    for (M, N) in [(0, 6), (5, 0)]:
        C, D = _run(lib, gi.make_problem(M, N, 3, "f32"))
        assert C.shape == (M, N)


def pin_nonnegative_scale(lib):
    """With nonnegative entries, D (sum of |products|) equals C bit for bit."""
    for dtype in DTYPES:
        p = gi.make_problem(19, 21, 300, dtype, dist="unit", wid=109)
        C, D = _run(lib, p)
        assert np.array_equal(C, D)


def pin_bf16_widening(lib):
    """bf16 bit patterns are read as the values they encode: 1.0 (0x3F80) times
    -2.5 (0xC020) plus 2^-126 (0x0080) times 3.0 (0x4040)."""
    A = np.array([0x3F80, 0x0080], dtype=np.uint16)   # 1 x 2 row-major
    B = np.array([0xC020, 0x4040], dtype=np.uint16)   # 2 x 1 row-major
    C, D = oracle.gemm(1, 1, 2, A, 2, ROW_MAJOR, B, 1, ROW_MAJOR, lib=lib)
    assert C[0, 0] == -2.5 + 3.0 * 2.0 ** -126
    assert D[0, 0] == 2.5 + 3.0 * 2.0 ** -126


def pin_f16_widening(lib):
    """Every IEEE binary16 bit pattern is read as the value it encodes, checked against
    numpy's own float16 -> float64 conversion (a library routine the oracle does not call)
    for all 65536 patterns: a 65536 x 1 times 1 x 1 product with B = 1 returns them."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    A = bits.view(np.float16)                          # 65536 x 1, row-major
    B = np.array([1.0], dtype=np.float16)
    C, D = oracle.gemm(65536, 1, 1, A, 1, ROW_MAJOR, B, 1, ROW_MAJOR, lib=lib)
    want = A.astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(C[:, 0]), nan)
    assert np.array_equal(C[~nan, 0], want[~nan])
    # spot values fixed by the format: 1.0 = 0x3C00, -2 = 0xC000, 65504 (largest) = 0x7BFF,
    # 2^-24 (smallest subnormal) = 0x0001, 2^-14 (smallest normal) = 0x0400, inf = 0x7C00
    for pattern, value in ((0x3C00, 1.0), (0xC000, -2.0), (0x7BFF, 65504.0), (0x0001, 2.0 ** -24),
                           (0x0400, 2.0 ** -14), (0x7C00, np.inf), (0x8000, -0.0)):
        assert C[pattern, 0] == value


def pin_fp8_widening(lib):
    """Every bit pattern of both OCP 8-bit formats is read as the value it encodes, checked
    against torch's float8_e4m3fn / float8_e5m2 -> float32 conversion (a library routine the
    oracle does not call) for all 256 patterns: a 256 x 1 times 1 x 1 product with B = 1 returns
    them.  Also the formats' fixed points: the largest finite values (448 = 0x7E, 57344 = 0x7B),
    the smallest subnormals (2^-9 = 0x01, 2^-16 = 0x01) and normals (2^-6 = 0x08, 2^-14 = 0x04),
    1.0 (0x38, 0x3C), -0 (0x80), E4M3's only NaNs 0x7F / 0xFF and E5M2's infinities 0x7C / 0xFC."""
    import torch
    bits = np.arange(256, dtype=np.uint16).astype(np.uint8)
    for fmt, tdt, one in (("e4m3", torch.float8_e4m3fn, 0x38), ("e5m2", torch.float8_e5m2, 0x3C)):
        B = np.array([one], dtype=np.uint8)
        C, D = oracle.gemm(256, 1, 1, bits, 1, ROW_MAJOR, B, 1, ROW_MAJOR, lib=lib, fmt_a=fmt, fmt_b=fmt)
        want = torch.from_numpy(bits.copy()).view(tdt).float().numpy().astype(np.float64)
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(C[:, 0]), nan), fmt
        assert np.array_equal(C[~nan, 0], want[~nan]), fmt
    C4, _ = oracle.gemm(256, 1, 1, bits, 1, ROW_MAJOR, np.array([0x38], np.uint8), 1, ROW_MAJOR, lib=lib,
                        fmt_a="e4m3", fmt_b="e4m3")
    for pattern, value in ((0x7E, 448.0), (0x01, 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0), (0xB8, -1.0),
                           (0x80, -0.0), (0x77, 240.0)):
        assert C4[pattern, 0] == value, (hex(pattern), C4[pattern, 0])
    assert np.isnan(C4[0x7F, 0]) and np.isnan(C4[0xFF, 0]) and np.isfinite(C4[0x78, 0])
    C5, _ = oracle.gemm(256, 1, 1, bits, 1, ROW_MAJOR, np.array([0x3C], np.uint8), 1, ROW_MAJOR, lib=lib,
                        fmt_a="e5m2", fmt_b="e5m2")
    for pattern, value in ((0x7B, 57344.0), (0x01, 2.0 ** -16), (0x04, 2.0 ** -14), (0x3C, 1.0),
                           (0x7C, np.inf), (0xFC, -np.inf), (0x80, -0.0)):
        assert C5[pattern, 0] == value, (hex(pattern), C5[pattern, 0])
    assert np.isnan(C5[0x7D, 0]) and np.isnan(C5[0xFF, 0])
    # mixed formats: an E4M3 A against an E5M2 B reads each in its own format
    C, _ = oracle.gemm(1, 1, 1, np.array([0x7E], np.uint8), 1, ROW_MAJOR, np.array([0x7B], np.uint8), 1,
                       ROW_MAJOR, lib=lib, fmt_a="e4m3", fmt_b="e5m2")
    assert C[0, 0] == 448.0 * 57344.0


def pin_sampled_matches_full(lib):
    """The sampled entry point returns the full product's elements bit for bit."""
    for dtype in DTYPES:
        for oa, ob in ORDERS:
            p = gi.make_problem(29, 33, 77, dtype, oa, ob, wid=110, pad_a=1)
            C, D = _run(lib, p)
            rng = np.random.default_rng(19)
            rows = rng.integers(0, p.M, 50)
            cols = rng.integers(0, p.N, 50)
            Cs, Ds = oracle.gemm_sampled(p.M, p.N, p.K, p.A, p.lda, p.order_a, p.B, p.ldb,
                                         p.order_b, rows, cols, lib=lib, **gi.oracle_formats(p))
            assert np.array_equal(Cs, C[rows, cols]) and np.array_equal(Ds, D[rows, cols])


def _batched(lib, p: gi.BatchedProblem):
    return oracle.gemm_strided_batched(p.batch, p.M, p.N, p.K, p.A, p.lda, p.sa, p.order_a, p.B, p.ldb,
                                       p.sb, p.order_b, lib=lib)


# layouts of a strided batch: interleaved rows ([rows, entries, cols]), stacked with gaps,
# and one operand shared by every entry (stride 0)
BATCH_LAYOUTS = [
    dict(lda=3 * 4, sa=4, ldb=5, sb=4 * 5 + 2),                  # A interleaved, B stacked + gap
    dict(order_a=COL_MAJOR, lda=2, sa=2 * 4 + 1, order_b=COL_MAJOR, ldb=3 * 4, sb=4),
    dict(sa=0, ldb=5 + 1),                                       # one A for every entry
    dict(order_a=COL_MAJOR, sb=0, order_b=COL_MAJOR),            # one B for every entry
]


def pin_batched_bruteforce(lib):
    """Each entry of a strided batch equals the exact rational product of that entry's own
    logical matrices (the generator's arrays, independent of the layout), for interleaved,
    stacked and shared operands."""
    for dtype in BATCH_DTYPES:
        for lay in BATCH_LAYOUTS:
            p = gi.make_batched_problem(3, 2, 5, 4, dtype, wid=111, **lay)
            C, D = _batched(lib, p)
            a = gi._to_f32(p.A_logical, dtype)
            b = gi._to_f32(p.B_logical, dtype)
            assert C.shape == (3, 2, 5)
            for z in range(3):
                for i in range(2):
                    for j in range(5):
                        exact = sum((Fraction(float(a[z, i, k])) * Fraction(float(b[z, k, j])) for k in range(4)),
                                    Fraction(0))
                        assert abs(Fraction(C[z, i, j]) - exact) <= Fraction(3, 2 ** 53) * Fraction(D[z, i, j])


def pin_batched_scaled_identity(lib):
    """A_z = (z + 1) I gives C_z = (z + 1) B_z exactly, entry by entry; an entry that read
    another entry's A or B, or the wrong stride, shows up as a wrong scale or matrix."""
    batch, n, N = 5, 6, 7
    eye = np.stack([(z + 1) * np.eye(n, dtype=np.float32) for z in range(batch)])
    rng = np.random.default_rng(23)
    Bl = _int_matrix(rng, batch * n, N).reshape(batch, n, N)
    for dtype in BATCH_DTYPES:
        for lay in (dict(), dict(lda=batch * n, sa=n, ldb=N + 3, sb=(N + 3) * n + 1)):
            p = gi.make_batched_problem(batch, n, N, n, dtype, A_logical=eye, B_logical=Bl, **lay)
            C, _ = _batched(lib, p)
            for z in range(batch):
                assert np.array_equal(C[z], (z + 1) * Bl[z].astype(np.float64))


def pin_epilogue_closed_forms(lib):
    """act(alpha*C + beta*C_old + bias) on small integers, exact in float64: identity with the
    defaults, scaling, the old C term, a bias per column (distinct values on a non-square C),
    ReLU, and beta == 0 never reading C_old (NaN there stays out)."""
    rng = np.random.default_rng(29)
    p = gi.make_problem(5, 7, 9, "f32", A_logical=_int_matrix(rng, 5, 9), B_logical=_int_matrix(rng, 9, 7))
    C, D = _run(lib, p)
    old = _int_matrix(rng, 5, 7)
    bias = np.arange(7, dtype=np.float64) * 3 - 10
    Y, _ = oracle.epilogue(C, D)
    assert np.array_equal(Y, C)
    Y, _ = oracle.epilogue(C, D, alpha=2.0, beta=-0.5, C_old=old, bias=bias)
    for i in range(5):
        for j in range(7):
            assert Y[i, j] == 2 * C[i, j] - 0.5 * old[i, j] + (3 * j - 10)
    Y, _ = oracle.epilogue(C, D, bias=bias, activation=oracle.ACT_RELU)
    assert np.array_equal(Y, np.where(C + bias > 0, C + bias, 0.0))
    Y, _ = oracle.epilogue(C, D, beta=0.0, C_old=np.full((5, 7), np.nan))
    assert np.array_equal(Y, C)


def pin_gelu_values(lib):
    """GELU(x) = x Phi(x): Phi(1) = 0.8413447460685429 and Phi(-1) = 0.15865525393145707 (the
    normal table), GELU(0) = 0, GELU(10) = 10 in float64, GELU(x) - GELU(-x) = x (Phi(x) +
    Phi(-x) = 1), and GELU of a large negative value vanishes (-10 Phi(-10) is about -8e-23)."""
    x = np.array([[1.0, -1.0, 0.0, 10.0, -10.0]])
    Y, _ = oracle.epilogue(x, np.abs(x), activation=oracle.ACT_GELU)
    assert abs(Y[0, 0] - 0.8413447460685429) < 1e-15
    assert abs(Y[0, 1] + 0.15865525393145707) < 1e-15
    assert Y[0, 2] == 0.0 and Y[0, 3] == 10.0 and abs(Y[0, 4]) < 1e-20
    r = np.random.default_rng(31).uniform(-6, 6, (1, 200))
    Yp, _ = oracle.epilogue(r, np.abs(r), activation=oracle.ACT_GELU)
    Yn, _ = oracle.epilogue(-r, np.abs(r), activation=oracle.ACT_GELU)
    assert np.allclose(Yp - Yn, r, rtol=0, atol=1e-14)


ALL_PINS = [
    pin_fraction_bruteforce, pin_numpy_crosscheck, pin_ones, pin_ones_column_sums,
    pin_identity, pin_permutation, pin_small_integers, pin_transpose, pin_k_split,
    pin_mac_count, pin_degenerate, pin_nonnegative_scale, pin_bf16_widening,
    pin_f16_widening, pin_fp8_widening, pin_sampled_matches_full, pin_batched_bruteforce, pin_batched_scaled_identity,
    pin_epilogue_closed_forms, pin_gelu_values,
]
