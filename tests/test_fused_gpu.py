"""Parity of the fused-epilogue entry points: C = act(alpha A.B + beta C + bias) in FP32 or
bf16, against the oracle's product followed by its epilogue, element by element."""
import numpy as np
import pytest

import gemm_f32_amd as g
import gemm_inputs as gi
import oracle
from gemm_inputs import COL_MAJOR as C_, ROW_MAJOR as R
from gpu_util import TOL, to_device

pytestmark = pytest.mark.gpu

BF16_NAN = np.uint16(0x7FC1)
# (alpha, beta, bias?, activation, output)
EPILOGUES = {
    "plain": (1.0, 0.0, False, g.Act.NONE, g.Out.F32),
    "scale_beta_bias_relu": (0.5, 2.0, True, g.Act.RELU, g.Out.F32),
    "bias_gelu_bf16": (1.0, 0.0, True, g.Act.GELU, g.Out.BF16),
    "beta_gelu_bf16": (-1.5, 1.0, False, g.Act.GELU, g.Out.BF16),
    "beta_bias_bf16": (1.0, 0.25, True, g.Act.NONE, g.Out.BF16),
}
SHAPES = [(300, 260, 96), (512, 512, 64), (77, 1030, 128), (1000, 700, 1000)]


def run_fused(p, epi, seed=0):
    """(got Y as float64 M x N, reference Y, scale S, untouched-padding flag)."""
    import torch
    alpha, beta, has_bias, act, out = epi
    rng = np.random.default_rng(seed)
    bias = rng.uniform(-1, 1, p.N).astype(np.float32) if has_bias else None
    old = rng.uniform(-1, 1, (p.M, p.N)).astype(np.float32)
    if out == g.Out.BF16:
        old_bits = gi.f32_to_bf16_bits(old)
        old = gi.bf16_bits_to_f32(old_bits)
        flat, _ = gi.lay_out(old_bits, p.order_c, p.ldc)
    else:
        flat, _ = gi.lay_out(old, p.order_c, p.ldc)
    if beta == 0.0:
        flat = np.full_like(flat, BF16_NAN if out == g.Out.BF16 else np.nan)   # never read
    A, B, C = to_device(p.A), to_device(p.B), to_device(flat)
    bias_d = to_device(bias) if bias is not None else None
    fn = {"bf16": g.gemm_bf16_f32acc_fused, "f16": g.gemm_f16_f32acc_fused, "f32": g.gemm_f32_fused}[p.dtype]
    print(f"[gpu] fused {p.dtype} M={p.M} N={p.N} K={p.K} oc={p.order_c} epi={epi}", flush=True)
    fn(p.M, p.N, p.K, A.data_ptr(), p.lda, p.order_a, B.data_ptr(), p.ldb, p.order_b, C.data_ptr(), p.ldc,
       p.order_c, alpha=alpha, beta=beta, bias=bias_d.data_ptr() if bias_d is not None else 0, activation=act,
       out_type=out, stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    res = C.cpu().numpy()
    if out == g.Out.BF16:
        res = res.view(np.uint16)
        got = gi.bf16_bits_to_f32(gi.unpack_c(res, p.M, p.N, p.ldc, p.order_c).copy())
        inner = p.N if p.order_c == R else p.M
        pad_ok = bool(np.all(res.reshape(-1, p.ldc)[:, inner:] == BF16_NAN)) if p.M and p.N else True
    else:
        got = gi.unpack_c(res, p.M, p.N, p.ldc, p.order_c)
        inner = p.N if p.order_c == R else p.M
        pad_ok = bool(np.all(np.isnan(res.reshape(-1, p.ldc)[:, inner:]))) if p.M and p.N else True
    ref, D = oracle.gemm(p.M, p.N, p.K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b)
    Y, S = oracle.epilogue(ref, D, alpha, beta, old, bias, int(act))
    return got.astype(np.float64), Y, S, pad_ok


def assert_close(got, Y, S, dtype, out):
    """|got - Y| <= TOL * S, plus 2^-8 |Y| for a bf16 output (its rounding, twice the half ulp)."""
    assert np.all(np.isfinite(got))
    bound = TOL[dtype] * S + (2.0 ** -8 * np.abs(Y) if out == g.Out.BF16 else 0.0)
    excess = np.abs(got - Y) - bound
    assert excess.max() <= 0, f"worst excess {excess.max():.3e} at {np.unravel_index(excess.argmax(), excess.shape)}"


@pytest.mark.parametrize("epi", list(EPILOGUES))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("oc", [R, C_], ids=["rowC", "colC"])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_fused_matches_oracle(dtype, oc, shape, epi):
    M, N, K = shape
    p = gi.make_problem(M, N, K, dtype, R, C_, oc, wid=81, pad_c=3)
    got, Y, S, pad_ok = run_fused(p, EPILOGUES[epi], seed=M + N)
    assert pad_ok, "C written outside the logical matrix"
    # the identity epilogue runs the plain kernel (16-bit inputs: on the same plan; FP32: gemm_f32)
    kernel = g.gemm_last_kernel()
    assert kernel.endswith("_fused") != (epi == "plain"), kernel
    if dtype != "f32" or epi != "plain":
        assert "_dma" in kernel, kernel
    assert_close(got, Y, S, dtype, EPILOGUES[epi][4])


@pytest.mark.parametrize("epi", ["scale_beta_bias_relu", "beta_gelu_bf16"])
def test_fused_empty_sum(epi):
    """K == 0: C = act(beta C + bias)."""
    p = gi.make_problem(70, 90, 0, "bf16", R, C_, R, pad_c=2)
    got, Y, S, pad_ok = run_fused(p, EPILOGUES[epi], seed=3)
    assert pad_ok and g.gemm_last_kernel() == "epilogue_fill"
    assert_close(got, Y, S, "bf16", EPILOGUES[epi][4])


def test_fused_relu_of_exact_products_is_exact():
    """Small-integer operands: the product is exact in FP32, so alpha = 1, ReLU and an integer
    bias give exactly the oracle's values, including the zeros ReLU makes."""
    rng = np.random.default_rng(9)
    Al = rng.integers(-4, 5, (260, 128)).astype(np.float32)
    Bl = rng.integers(-4, 5, (128, 300)).astype(np.float32)
    p = gi.make_problem(260, 300, 128, "bf16", R, C_, R, A_logical=Al, B_logical=Bl)
    import torch
    bias = np.arange(300, dtype=np.float32) % 7 - 3
    C = torch.full((p.M * p.ldc,), float("nan"), dtype=torch.float32, device="cuda")
    A, B, bias_d = to_device(p.A), to_device(p.B), to_device(bias)    # held until the call has run
    g.gemm_bf16_f32acc_fused(p.M, p.N, p.K, A.data_ptr(), p.lda, R, B.data_ptr(), p.ldb, C_, C.data_ptr(), p.ldc,
                             R, bias=bias_d.data_ptr(), activation=g.Act.RELU)
    torch.cuda.synchronize()
    want = np.maximum(Al.astype(np.float64) @ Bl + bias, 0)
    assert np.array_equal(C.cpu().numpy().reshape(p.M, p.N), want)


def test_fused_ffn_up_full_size_sampled():
    """LLaMA-2-7B FFN-up (2048 x 11008 x 4096) with bias, GELU and a bf16 output, sampled."""
    import torch
    from test_workloads_gpu import sample_indices
    p = gi.workload_problem("llm_ffn_up_2048x11008x4096")
    rng = np.random.default_rng(17)
    bias = rng.uniform(-1, 1, p.N).astype(np.float32)
    C = torch.full((p.M * p.ldc,), -1, dtype=torch.int16, device="cuda")
    print("[gpu] fused ffn-up full size", flush=True)
    A, B, bias_d = to_device(p.A), to_device(p.B), to_device(bias)    # held until the call has run
    g.gemm_bf16_f32acc_fused(p.M, p.N, p.K, A.data_ptr(), p.lda, R, B.data_ptr(), p.ldb, C_, C.data_ptr(), p.ldc,
                             R, bias=bias_d.data_ptr(), activation=g.Act.GELU, out_type=g.Out.BF16)
    torch.cuda.synchronize()
    got = gi.bf16_bits_to_f32(C.cpu().numpy().view(np.uint16)).reshape(p.M, p.N).astype(np.float64)
    rows, cols = sample_indices(p.M, p.N, 5)
    ref, D = oracle.gemm_sampled(p.M, p.N, p.K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b, rows, cols)
    Y, S = oracle.epilogue(ref[None, :], D[None, :], bias=bias[cols], activation=oracle.ACT_GELU)
    assert_close(got[rows, cols][None, :], Y, S, "bf16", g.Out.BF16)


@pytest.mark.parametrize("oc", [R, C_], ids=["rowC", "colC"])
def test_fused_ffn_up_core_and_strip(oc):
    """2048 x 11008 x 4096 runs as a 256 x 256 core and a 256 x 128 strip (along N for a row-major
    C, along the normalised M for a column-major one): beta, bias and ReLU, sampled outputs on both
    sides of the seam against the oracle."""
    import torch
    from test_workloads_gpu import sample_indices
    p = gi.workload_problem("llm_ffn_up_2048x11008x4096")
    if oc == C_:
        p = gi.make_problem(p.M, p.N, p.K, "bf16", R, C_, C_, A_logical=gi.bf16_bits_to_f32(p.A_logical),
                            B_logical=gi.bf16_bits_to_f32(p.B_logical))
    rng = np.random.default_rng(23)
    bias = rng.uniform(-1, 1, p.N).astype(np.float32)
    old = rng.uniform(-1, 1, (p.M, p.N)).astype(np.float32)
    flat, _ = gi.lay_out(old, p.order_c, p.ldc)
    A, B, C, bias_d = to_device(p.A), to_device(p.B), to_device(flat), to_device(bias)
    print(f"[gpu] fused ffn-up core and strip oc={oc}", flush=True)
    g.gemm_bf16_f32acc_fused(p.M, p.N, p.K, A.data_ptr(), p.lda, R, B.data_ptr(), p.ldb, C_, C.data_ptr(), p.ldc,
                             p.order_c, alpha=0.5, beta=1.0, bias=bias_d.data_ptr(), activation=g.Act.RELU)
    torch.cuda.synchronize()
    assert g.gemm_last_kernel() == "bf16_dma256x256_fused"
    got = gi.unpack_c(C.cpu().numpy(), p.M, p.N, p.ldc, p.order_c).astype(np.float64)
    rows, cols = sample_indices(p.M, p.N, 5)
    seam = 8192       # the strip's first column of C (a row of the normalised C when C is column-major)
    extra_c = np.arange(seam - 64, seam + 64)
    extra_r = rng.integers(0, p.M, extra_c.size)
    rows, cols = np.concatenate([rows, extra_r]), np.concatenate([cols, extra_c])
    ref, D = oracle.gemm_sampled(p.M, p.N, p.K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b, rows, cols)
    Y, S = oracle.epilogue(ref[None, :], D[None, :], alpha=0.5, beta=1.0, C_old=old[rows, cols][None, :],
                           bias=bias[cols], activation=oracle.ACT_RELU)
    assert_close(got[rows, cols][None, :], Y, S, "bf16", g.Out.F32)


@pytest.mark.parametrize("out", [g.Out.F32, g.Out.BF16], ids=["f32", "bf16"])
def test_fused_gelu_accuracy(out):
    """GELU on exact pre-activations: small-integer operands make every sum exact, alpha = 2^-5 maps
    them onto about [-8, 8].  FP32 output within 5e-7 |x| of x Phi(x) (the epilogue's erf is
    Abramowitz and Stegun 7.1.26, |error| <= 1.5e-7, evaluated with the hardware's exp2 and
    reciprocal; 3.0e-7 |x| at most in a float32 emulation with exact exp2 and reciprocal); a bf16
    output is that value rounded to nearest even, so within 2^-8 |y| + 5e-7 |x|."""
    import torch
    from scipy.special import erf
    rng = np.random.default_rng(31)
    M, N, K = 256, 384, 64
    Al = rng.integers(-4, 5, (M, K)).astype(np.float32)
    Bl = rng.integers(-4, 5, (K, N)).astype(np.float32)
    p = gi.make_problem(M, N, K, "bf16", R, C_, R, A_logical=Al, B_logical=Bl)
    alpha = 2.0 ** -5
    A, B = to_device(p.A), to_device(p.B)
    if out == g.Out.F32:
        C = torch.full((M * N,), float("nan"), dtype=torch.float32, device="cuda")
    else:
        C = torch.full((M * N,), -1, dtype=torch.int16, device="cuda")
    print(f"[gpu] fused gelu accuracy out={int(out)}", flush=True)
    g.gemm_bf16_f32acc_fused(M, N, K, A.data_ptr(), p.lda, R, B.data_ptr(), p.ldb, C_, C.data_ptr(), N, R,
                             alpha=alpha, activation=g.Act.GELU, out_type=out)
    torch.cuda.synchronize()
    res = C.cpu().numpy()
    got = (gi.bf16_bits_to_f32(res.view(np.uint16)) if out == g.Out.BF16 else res).reshape(M, N).astype(np.float64)
    x = alpha * (Al.astype(np.float64) @ Bl)
    assert np.abs(x).max() > 4
    ref = x * 0.5 * (1.0 + erf(x / np.sqrt(2.0)))
    bound = 5e-7 * np.abs(x) + (2.0 ** -8 * np.abs(ref) if out == g.Out.BF16 else 0.0)
    assert np.all(np.abs(got - ref) <= bound + 1e-30)


@pytest.mark.parametrize("oc", [R, C_], ids=["rowC", "colC"])
def test_f32_fused_whole_tiles_and_edges(oc):
    """FP32 inputs on 256 x 256 tiles overhanging both edges (4095 x 4097 x 512): beta, bias and
    ReLU, sampled on whole rows and columns at tile boundaries against the oracle."""
    import torch
    from test_workloads_gpu import sample_indices
    M, N, K = 4095, 4097, 512
    p = gi.make_problem(M, N, K, "f32", R, C_, oc, wid=82)
    rng = np.random.default_rng(29)
    bias = rng.uniform(-1, 1, N).astype(np.float32)
    old = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    flat, _ = gi.lay_out(old, p.order_c, p.ldc)
    A, B, C, bias_d = to_device(p.A), to_device(p.B), to_device(flat), to_device(bias)
    print(f"[gpu] f32 fused 4095x4097x512 oc={oc}", flush=True)
    g.gemm_f32_fused(M, N, K, A.data_ptr(), p.lda, R, B.data_ptr(), p.ldb, C_, C.data_ptr(), p.ldc, p.order_c,
                     alpha=0.75, beta=0.5, bias=bias_d.data_ptr(), activation=g.Act.RELU)
    torch.cuda.synchronize()
    assert g.gemm_last_kernel() == "f32_dma256x256_fused"
    got = gi.unpack_c(C.cpu().numpy(), M, N, p.ldc, p.order_c).astype(np.float64)
    rows, cols = sample_indices(M, N, 7)
    ref, D = oracle.gemm_sampled(M, N, K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b, rows, cols)
    Y, S = oracle.epilogue(ref[None, :], D[None, :], alpha=0.75, beta=0.5, C_old=old[rows, cols][None, :],
                           bias=bias[cols], activation=oracle.ACT_RELU)
    assert_close(got[rows, cols][None, :], Y, S, "f32", g.Out.F32)


# --- row-major B (n-contiguous, PyTorch's x . W with W [K, N]): the direct-copy kernel keeps the B
# k-tile as laid out and reads it with gfx950's transposing LDS read; N % 8 == 0 --------------------
BRM_SHAPES = [(300, 264, 96), (512, 512, 64), (77, 1032, 128), (1000, 704, 1000)]


@pytest.mark.parametrize("epi", list(EPILOGUES))
@pytest.mark.parametrize("shape", BRM_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("orders", [(R, R, R), (C_, C_, C_)], ids=["RRR", "CCC"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fused_row_major_b_matches_oracle(dtype, orders, shape, epi):
    """All three operands row-major, or all three column-major (C^T = B^T A^T turns it into the
    same row-major-B problem): every epilogue against the oracle, C's padding untouched."""
    M, N, K = shape
    oa, ob, oc = orders
    if oc == C_:
        M, N = N, M                 # the swapped problem's N is this problem's M: keep it % 8 == 0
    p = gi.make_problem(M, N, K, dtype, oa, ob, oc, wid=83, pad_c=3)
    got, Y, S, pad_ok = run_fused(p, EPILOGUES[epi], seed=M + 2 * N)
    assert pad_ok, "C written outside the logical matrix"
    kernel = g.gemm_last_kernel()
    assert "_dma" in kernel and kernel.endswith("_fused") != (epi == "plain"), kernel
    assert_close(got, Y, S, dtype, EPILOGUES[epi][4])


@pytest.mark.parametrize("case", ["RRC", "N%8"])
def test_fused_refuses_layouts_the_kernel_does_not_take(case):
    """Row-major A and B with a column-major C (the swap makes A column-major), and row-major B with
    N % 8 != 0: refused before anything is enqueued, C left as it was."""
    import torch
    if case == "RRC":
        p = gi.make_problem(128, 256, 64, "bf16", R, R, C_)
    else:
        p = gi.make_problem(128, 260, 64, "bf16", R, R, R)
    A, B = to_device(p.A), to_device(p.B)
    C = torch.full((gi.c_buffer_size(p.M, p.N, p.ldc, p.order_c),), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(g.GemmError) as e:
        g.gemm_bf16_f32acc_fused(p.M, p.N, p.K, A.data_ptr(), p.lda, p.order_a, B.data_ptr(), p.ldb, p.order_b,
                                 C.data_ptr(), p.ldc, p.order_c, alpha=2.0, activation=g.Act.RELU)
    assert e.value.status == g.Status.ERR_INVALID_VALUE
    torch.cuda.synchronize()
    assert torch.all(C == 7.0).item()
