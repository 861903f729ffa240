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


@pytest.mark.parametrize("name", [n for n, w in gi.WORKLOADS.items() if w.batch == 1])
def test_workload_full_size_sampled(name):
    p = gi.workload_problem(name)
    flat = run(p)
    assert padding_untouched(p, flat)
    C = logical_c(p, flat)
    assert np.all(np.isfinite(C)), "every output written and finite"
    rows, cols = sample_indices(p.M, p.N, gi.WORKLOADS[name].wid)
    ref, D = oracle.gemm_sampled(p.M, p.N, p.K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b,
                                 rows, cols, **gi.oracle_formats(p))
    err = oracle.normalised_error(C[rows, cols], ref, D)
    print(f"{name}: normalised error {err:.3e} over {rows.size} sampled outputs")
    assert err <= TOL[p.dtype]


# the workloads whose default plan splits K when given a workspace
WS_WORKLOADS = [n for n in gi.WORKLOADS if n.startswith(("fewcols", "shard"))] + ["llm_ffn_down_2048x4096x11008"]


@pytest.mark.parametrize("name", WS_WORKLOADS)
def test_workload_full_size_sampled_with_workspace(name):
    """The workspace entry point (split-K across workgroups) at the workload's full size."""
    import torch
    import gemm_f32_amd as g
    from gpu_util import to_device
    p = gi.workload_problem(name)
    need = g.gemm_workspace_size(p.dtype, p.M, p.N, p.K, p.order_a, p.order_b, p.order_c)
    assert need > 0
    A, B = to_device(p.A), to_device(p.B)
    C = torch.full((gi.c_buffer_size(p.M, p.N, p.ldc, p.order_c),), float("nan"), dtype=torch.float32,
                   device="cuda")
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    fn = {"f32": g.gemm_f32_ws, "bf16": g.gemm_bf16_f32acc_ws, "f16": g.gemm_f16_f32acc_ws}[p.dtype]
    print(f"[gpu] ws workload {name}", flush=True)
    fn(p.M, p.N, p.K, A.data_ptr(), p.lda, p.order_a, B.data_ptr(), p.ldb, p.order_b, C.data_ptr(), p.ldc,
       p.order_c, ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert g.gemm_last_kernel().endswith("_splitk")
    flat = C.cpu().numpy()
    assert padding_untouched(p, flat)
    Cl = logical_c(p, flat)
    assert np.all(np.isfinite(Cl))
    rows, cols = sample_indices(p.M, p.N, gi.WORKLOADS[name].wid)
    ref, D = oracle.gemm_sampled(p.M, p.N, p.K, p.A, p.lda, p.order_a, p.B, p.ldb, p.order_b, rows, cols)
    err = oracle.normalised_error(Cl[rows, cols], ref, D)
    print(f"{name} (workspace): normalised error {err:.3e} over {rows.size} sampled outputs")
    assert err <= TOL[p.dtype]


@pytest.mark.parametrize("name", [n for n, w in gi.WORKLOADS.items() if w.batch > 1])
def test_batched_workload_full_size_sampled(name):
    """Strided batch at full size: sampled outputs of the first, second, a middle and the last
    entry, each from the oracle on that entry's operands."""
    from gpu_util import run_batched
    p = gi.workload_problem(name)
    flat = run_batched(p)
    got = p.c_view(flat)
    assert np.all(np.isfinite(got)), "every output written and finite"
    assert np.all(np.isnan(p.c_untouched(flat)))
    for z in sorted({0, 1, p.batch // 2, p.batch - 1}):
        rows, cols = sample_indices(p.M, p.N, gi.WORKLOADS[name].wid + z)
        ref, D = oracle.gemm_sampled(p.M, p.N, p.K, p.A[z * p.sa:], p.lda, p.order_a, p.B[z * p.sb:], p.ldb,
                                     p.order_b, rows, cols)
        err = oracle.normalised_error(got[z][rows, cols], ref, D)
        print(f"{name} entry {z}: normalised error {err:.3e} over {rows.size} sampled outputs")
        assert err <= TOL[p.dtype]
