"""Library calls captured into a HIP graph (torch.cuda.CUDAGraph on the capture stream).

The plain calls allocate nothing and record no memset (C is zeroed by a kernel where a path
needs it), so a caller can capture them.  Each case runs the call eagerly, captures the same
call, then replays the graph several times with eager work and synchronisations between the
replays, C reset to NaN before each; every replay must reproduce the eager result bit for bit
(every kernel on these paths is deterministic)."""
import numpy as np
import pytest

import gemm_f32_amd as g
import gemm_inputs as gi
from gemm_inputs import COL_MAJOR, ROW_MAJOR
from gpu_util import to_device

pytestmark = pytest.mark.gpu

CASES = [
    # few FP32 rows: the two-halves mode (a zero-fill kernel, then the two K halves' atomic adds)
    ("f32", (16, 4096, 4096), ROW_MAJOR, "f32_skinny32_halves"),
    # the small-problem kernel's 64 x 64 blocks, the FP32 and BF16 direct-copy kernels, a ragged
    # shape with an edge strip, the K = 0 fill
    ("f32", (1024, 1024, 1024), ROW_MAJOR, "f32_skinny64"),
    ("bf16", (1024, 1024, 512), COL_MAJOR, "bf16_skinny64"),
    ("f32", (2048, 2048, 256), ROW_MAJOR, "f32_dma"),
    ("bf16", (2048, 4096, 128), COL_MAJOR, "bf16_dma"),
    ("f32", (1000, 1030, 257), ROW_MAJOR, None),
    ("f32", (300, 200, 0), ROW_MAJOR, "zero_c"),
]


@pytest.mark.parametrize("dtype,shape,ob,kernel", CASES, ids=lambda v: str(v))
def test_graph_replays_match_eager(dtype, shape, ob, kernel):
    import torch
    M, N, K = shape
    p = gi.make_problem(M, N, K, dtype, ROW_MAJOR, ob, wid=80)
    A, B = to_device(p.A), to_device(p.B)
    C = torch.full((gi.c_buffer_size(p.M, p.N, p.ldc, p.order_c),), float("nan"), dtype=torch.float32,
                   device="cuda")
    fn = g.gemm_f32 if dtype == "f32" else g.gemm_bf16_f32acc

    def call():
        fn(M, N, K, A.data_ptr(), p.lda, p.order_a, B.data_ptr(), p.ldb, p.order_b, C.data_ptr(), p.ldc,
           p.order_c, torch.cuda.current_stream().cuda_stream)

    print(f"[gpu] graph {dtype} M={M} N={N} K={K}", flush=True)
    call()
    torch.cuda.synchronize()
    eager = C.clone()
    assert not torch.isnan(eager).any()
    if kernel is not None:
        assert g.gemm_last_kernel().startswith(kernel)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    for replay in range(4):
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        # the program's own eager work between replays
        x = torch.from_numpy(rng.standard_normal(1 << 18).astype(np.float32)).cuda()
        assert torch.isfinite((x * 2.0).cumsum(0)).all()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(C.view(torch.int32), eager.view(torch.int32)), f"replay {replay} differs from the eager call"
