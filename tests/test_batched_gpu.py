"""Parity of the strided batched entry points with the oracle, entry by entry, on the GPU.

Layouts cover what attention's per-head products use (heads interleaved in the rows of a
[tokens, heads, head_dim] tensor, score matrices stacked per head), stacked entries with gaps,
one operand shared by every entry (stride 0), column-major C, ragged shapes over several
tiles, K == 0 and a batch larger than one launch covers."""
import numpy as np
import pytest

import gemm_f32_amd as g
import gemm_inputs as gi
from gemm_inputs import COL_MAJOR as C_, ROW_MAJOR as R
from gpu_util import check_batched

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "bf16", "f16"]

# (batch, M, N, K, orders (a, b, c), layout)
CASES = {
    "small_rows_rc": (5, 40, 72, 200, (R, C_, R), {}),
    "small_rows_rr": (4, 16, 100, 130, (R, R, R), {}),
    "ragged_rc": (3, 300, 260, 96, (R, C_, R), {}),
    "ragged_rr": (3, 300, 260, 96, (R, R, R), {}),
    "ragged_cc_colc": (2, 130, 200, 70, (C_, C_, C_), {}),
    "whole_tiles_rc": (2, 512, 512, 64, (R, C_, R), {}),
    "whole_tiles_rr": (2, 512, 256, 128, (R, R, R), {}),
    "core_and_strips": (2, 520, 1030, 64, (R, C_, R), {}),
    # attention at 320 tokens, 4 heads of 64: Q.K^T and P.V
    "scores_heads": (4, 320, 320, 64, (R, C_, R), dict(lda=256, sa=64, ldb=256, sb=64)),
    "pv_heads": (4, 320, 64, 320, (R, R, R), dict(ldb=256, sb=64, ldc=256, sc=64)),
    "gaps_and_padding": (3, 70, 90, 110, (R, C_, R), dict(lda=113, sa=113 * 70 + 7, ldb=111,
                                                           sb=111 * 90 + 5, ldc=93, sc=93 * 70 + 3)),
    "shared_a": (3, 96, 160, 80, (R, C_, R), dict(sa=0)),
    "shared_b": (3, 96, 160, 80, (R, R, R), dict(sb=0)),
    "col_c_interleaved": (3, 64, 40, 72, (R, C_, C_), dict(ldc=3 * 64, sc=64)),
    "k_zero": (3, 33, 17, 0, (R, R, R), {}),
}


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("dtype", DTYPES)
def test_batched_matches_oracle(dtype, case):
    batch, M, N, K, (oa, ob, oc), lay = CASES[case]
    p = gi.make_batched_problem(batch, M, N, K, dtype, oa, ob, oc, wid=71, **lay)
    check_batched(p)
    if K == 0:
        assert g.gemm_last_kernel() == "zero_c"
    else:
        assert g.gemm_last_kernel().startswith(dtype + "_")


@pytest.mark.parametrize("dtype", DTYPES)
def test_batch_of_one_is_the_plain_call(dtype):
    p = gi.make_batched_problem(1, 200, 136, 72, dtype, R, C_, R, sa=12345, sb=0, sc=0)
    check_batched(p)


def test_batch_beyond_one_launch():
    """70000 entries of 4 x 4 x 4: two launches of the grid's z extent."""
    p = gi.make_batched_problem(70000, 4, 4, 4, "f32", wid=72)
    check_batched(p)


def test_identity_entries_scale_exactly():
    """A_z = (z + 1) I: every entry of C is exactly (z + 1) B_z, so an entry that read another
    entry's operands or wrote another entry's C is caught exactly."""
    batch, n, N = 6, 96, 160
    eye = np.stack([(z + 1) * np.eye(n, dtype=np.float32) for z in range(batch)])
    rng = np.random.default_rng(5)
    Bl = rng.integers(-8, 9, size=(batch, n, N)).astype(np.float32)
    for dtype in DTYPES:
        p = gi.make_batched_problem(batch, n, N, n, dtype, R, C_, R, A_logical=eye, B_logical=Bl)
        from gpu_util import run_batched
        got = p.c_view(run_batched(p))
        want = (np.arange(1, batch + 1, dtype=np.float32)[:, None, None] * Bl)
        assert np.array_equal(got, want)
