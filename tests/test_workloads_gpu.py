"""Parity at the full sizes of the measured workloads, in the launch configuration the bench
times (the AUTO kernel choice).  The oracle computes sampled outputs one by one: whole rows
and columns at the start, middle, end and at tile boundaries (catching index and edge
mistakes), plus random elements."""
import numpy as np
import pytest

import gemm_inputs as gi
import oracle
from gpu_util import TOL, logical_c, padding_untouched, run

pytestmark = pytest.mark.gpu


def sample_indices(M, N, seed):
    rng = np.random.default_rng(seed)
    rows = sorted({r for r in (0, 1, 31, 32, 127, 128, 255, 256, M // 2, M - 2, M - 1) if 0 <= r < M})
    cols = sorted({c for c in (0, 1, 31, 32, 127, 128, 255, 256, N // 2, N - 2, N - 1) if 0 <= c < N})
    r = [np.full(N, i) for i in rows] + [np.arange(M) for _ in cols] + [rng.integers(0, M, 20000)]
    c = [np.arange(N) for _ in rows] + [np.full(M, j) for j in cols] + [rng.integers(0, N, 20000)]
    return np.concatenate(r), np.concatenate(c)


@pytest.mark.parametrize("name", list(gi.WORKLOADS))
def test_workload_full_size_sampled(name):
    p = gi.workload_problem(name)
    flat = run(p)
    assert padding_untouched(p, flat)
    C = logical_c(p, flat)
    assert np.all(np.isfinite(C)), "every output written and finite"
    rows, cols = sample_indices(p.M, p.N, gi.WORKLOADS[name].wid)
    ref, D = oracle.gemm_sampled(p.M, p.N, p.K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b,
                                 rows, cols)
    err = oracle.normalised_error(C[rows, cols], ref, D)
    print(f"{name}: normalised error {err:.3e} over {rows.size} sampled outputs")
    assert err <= TOL[p.dtype]
