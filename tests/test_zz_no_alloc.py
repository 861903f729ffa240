"""gemm_bf16_f32acc_noalloc: the workspace call with the library's static scratch instead of a
caller's workspace.  Its output must match gemm_bf16_f32acc_ws's (same kernels, same split, so
bit for bit) and the fp64 oracle within the BF16 tolerance, on two calls in a row, the second
smaller than the first (the scratch keeps the first call's partial sums)."""
import numpy as np
import pytest

import gemm_f32_amd as g
import gemm_inputs as gi
import oracle

from gpu_util import TOL, to_device

pytestmark = pytest.mark.gpu


def _call(fn, p, A, B, *ws):
    import torch
    C = torch.full((gi.c_buffer_size(p.M, p.N, p.ldc, p.order_c),), float("nan"), dtype=torch.float32,
                   device="cuda")
    fn(p.M, p.N, p.K, A.data_ptr(), p.lda, p.order_a, B.data_ptr(), p.ldb, p.order_b, C.data_ptr(), p.ldc,
       p.order_c, *ws, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return C.cpu().numpy(), g.gemm_last_kernel()


# (M, N, K): shapes whose output gives too few workgroups, so both calls split K across
# workgroups through the workspace; the second is smaller than the first
SHAPES = [(16, 1024, 16384), (8, 512, 8192)]


def test_noalloc_matches_workspace_call_twice_in_a_row():
    import torch
    for i, (M, N, K) in enumerate(SHAPES):
        p = gi.make_problem(M, N, K, "bf16", gi.ROW_MAJOR, gi.COL_MAJOR, wid=50 + i)
        need = g.gemm_workspace_size("bf16", M, N, K, p.order_a, p.order_b, p.order_c)
        assert 0 < need <= g.NOALLOC_SCRATCH_BYTES
        A, B = to_device(p.A), to_device(p.B)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        print(f"[gpu] noalloc vs ws bf16 M={M} N={N} K={K} workspace {need} B", flush=True)
        want, k_ws = _call(g.gemm_bf16_f32acc_ws, p, A, B, ws.data_ptr(), need)
        got, k_na = _call(g.gemm_bf16_f32acc_noalloc, p, A, B)
        assert k_ws.endswith("_splitk") and k_na == k_ws, (k_ws, k_na)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), "differs from the workspace call"
        ref, D = oracle.gemm(M, N, K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b)
        err = oracle.normalised_error(gi.unpack_c(got, M, N, p.ldc, p.order_c), ref, D)
        assert err <= TOL["bf16"], err


def test_noalloc_plain_shapes_and_empty_problems():
    """Shapes that do not split run the plain path; K == 0 zeroes C; M == 0 does nothing."""
    for M, N, K in [(300, 257, 129), (64, 64, 0)]:
        p = gi.make_problem(M, N, K, "bf16", gi.ROW_MAJOR, gi.COL_MAJOR, wid=60)
        A, B = to_device(p.A), to_device(p.B)
        got, _ = _call(g.gemm_bf16_f32acc_noalloc, p, A, B)
        ref, D = oracle.gemm(M, N, K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b)
        err = oracle.normalised_error(gi.unpack_c(got, M, N, p.ldc, p.order_c), ref, D)
        assert err <= TOL["bf16"], err
    p = gi.make_problem(0, 16, 16, "bf16", gi.ROW_MAJOR, gi.COL_MAJOR, wid=61)
    _call(g.gemm_bf16_f32acc_noalloc, p, to_device(p.A), to_device(p.B))
    assert g.gemm_last_kernel() == "none"


def test_noalloc_refuses_a_split_beyond_its_scratch():
    """2048 x 2048 x 8192 splits K into 4 slices: 3 slabs of 16 MiB exceed the 32 MiB scratch."""
    M, N, K = 2048, 2048, 8192
    need = g.gemm_workspace_size("bf16", M, N, K, gi.ROW_MAJOR, gi.COL_MAJOR, gi.ROW_MAJOR)
    assert need > g.NOALLOC_SCRATCH_BYTES
    import torch
    A = torch.zeros(M * K, dtype=torch.int16, device="cuda")
    B = torch.zeros(N * K, dtype=torch.int16, device="cuda")
    C = torch.zeros(M * N, dtype=torch.float32, device="cuda")
    with pytest.raises(g.GemmError) as e:
        g.gemm_bf16_f32acc_noalloc(M, N, K, A.data_ptr(), K, gi.ROW_MAJOR, B.data_ptr(), K, gi.COL_MAJOR,
                                   C.data_ptr(), N, gi.ROW_MAJOR, torch.cuda.current_stream().cuda_stream)
    assert e.value.status == g.Status.ERR_SCRATCH_TOO_SMALL
