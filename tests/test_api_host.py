"""Host-side checks of the C ABI (no kernel runs): exports, argument validation, the
tile scheduler and the torch-stride marshalling."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import gemm_f32_amd as g
from conftest import ROOT, gpu_available

HEADER = os.path.join(ROOT, "include", "gemm.h")
F32, BF16 = g.gemm_f32_algo, g.gemm_bf16_f32acc_algo
R, C_ = g.Order.ROW_MAJOR, g.Order.COL_MAJOR
INVALID = g.Status.ERR_INVALID_VALUE
FAKE = 1 << 20          # a non-null, aligned address; never dereferenced by these calls


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(g.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(g.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", g.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (gemm_\w+)$", out, flags=re.M))
    assert exported == set(declared_functions())


def test_strings():
    assert g.gemm_version() == "0.1.0"
    assert g.gemm_status_string(0) == "GEMM_OK"
    for s in (1, 2, 3):
        assert g.gemm_status_string(s).startswith(g.Status(s).name.replace("ERR", "GEMM_ERR", 1))
    assert "unknown" in g.gemm_status_string(99)


def _status(fn, *args, **kw):
    try:
        fn(*args, **kw)
    except g.GemmError as e:
        return e.status
    return g.Status.OK


def args(M=8, N=8, K=8, A=FAKE, lda=8, oa=R, B=FAKE, ldb=8, ob=R, C=FAKE, ldc=8, oc=R):
    return (M, N, K, A, lda, oa, B, ldb, ob, C, ldc, oc, 0)


@pytest.mark.parametrize("bad", [
    dict(M=-1), dict(N=-1), dict(K=-1), dict(M=2**31), dict(K=2**31),
    dict(lda=7), dict(oa=C_, lda=7), dict(ldb=7), dict(ob=C_, ldb=7), dict(ldc=7),
    dict(oc=C_, ldc=7), dict(lda=0, K=0), dict(oa=2), dict(ob=-1), dict(oc=5),
    dict(A=0), dict(B=0), dict(C=0), dict(C=FAKE + 2), dict(A=FAKE + 1),
], ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
@pytest.mark.parametrize("fn", [F32, BF16], ids=["f32", "bf16"])
def test_invalid_arguments_rejected_before_launch(fn, bad):
    if fn is BF16 and bad.get("A") == FAKE + 1:
        pytest.skip("odd address is 2-byte aligned: valid for bf16")
    assert _status(fn, g.Algo.AUTO, *args(**bad)) == INVALID


def fp8_args(M=8, N=8, K=8, A=FAKE, lda=8, oa=R, fa=0, B=FAKE, ldb=8, ob=C_, fb=0, C=FAKE, ldc=8, oc=R):
    return (M, N, K, A, lda, oa, fa, B, ldb, ob, fb, C, ldc, oc, 0)


@pytest.mark.parametrize("bad", [
    dict(M=-1), dict(K=-1), dict(K=2**31), dict(lda=7), dict(ldb=7), dict(ldc=7), dict(oc=C_, ldc=7),
    dict(oa=C_), dict(ob=R), dict(oa=C_, ob=R), dict(fa=2), dict(fb=-1), dict(A=0), dict(C=0),
    dict(C=FAKE + 2),
], ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_fp8_invalid_arguments_rejected_before_launch(bad):
    """8-bit operands: k-contiguous layouts only, two formats; any byte alignment of A and B."""
    assert _status(g.gemm_fp8_f32acc, *fp8_args(**bad)) == INVALID


def test_fp8_plan():
    assert g.gemm_plan("e4m3", 4096, 4096, 4096, R, C_, R) == ("fp8_dma256x256", 4096, 4096)
    assert g.gemm_plan("fp8", 256, 128, 384, R, C_, R)[0] == "fp8_dma256x128"
    # a column-major C swaps the roles: 16 x 4096 becomes 4096 x 16
    assert g.gemm_plan("fp8", 16, 4096, 4096, R, C_, C_) == ("fp8_dma256x128", 4096, 16)
    assert g.gemm_plan("fp8", 8, 8, 0, R, C_, R)[0] == "zero_c"
    assert g.gemm_plan("fp8", 64, 64, 64, R, C_, R, with_workspace=True)[3] == 0
    with pytest.raises(g.GemmError):
        g.gemm_plan("fp8", 64, 64, 64, C_, C_, R)


def test_f32_needs_4_byte_alignment_bf16_needs_2():
    assert _status(F32, g.Algo.AUTO, *args(A=FAKE + 2)) == INVALID
    assert _status(BF16, g.Algo.AUTO, *args(A=FAKE + 1)) == INVALID


@pytest.mark.parametrize("algo", [1, 2, 3, 4])
def test_bf16_rejects_vector_alu_ladder(algo):
    assert _status(BF16, algo, *args()) == INVALID


@pytest.mark.parametrize("algo", [7, 10, 13, -1])
def test_f32_rejects_unknown_tiles(algo):
    assert _status(F32, algo, *args()) == INVALID


@pytest.mark.parametrize("algo", [13, 100])
def test_bf16_rejects_unknown_algo(algo):
    assert _status(BF16, algo, *args()) == INVALID


@pytest.mark.parametrize("shape", [(0, 8, 8), (8, 0, 8), (0, 0, 0)])
def test_empty_output_is_ok_without_launch(shape):
    M, N, K = shape
    # nothing to do: no pointer is touched, no device is needed
    assert _status(F32, 0, *args(M, N, K, A=0, B=0, C=0, lda=max(K, 1), ldb=max(N, 1),
                                 ldc=max(N, 1))) == g.Status.OK
    assert g.gemm_last_kernel() == "none"


@pytest.mark.skipif(gpu_available(), reason="checks the no-GPU path")
def test_valid_call_without_gpu_reports_unsupported_device():
    assert _status(F32, 0, *args()) == g.Status.ERR_UNSUPPORTED_DEVICE


def test_operand_layout_from_torch_strides():
    torch = pytest.importorskip("torch")
    a = torch.empty(6, 10)
    assert g.operand_layout(a) == (10, R)
    assert g.operand_layout(a.t()) == (10, C_)
    assert g.operand_layout(torch.empty(6, 16)[:, :10]) == (16, R)
    assert g.operand_layout(torch.empty(10, 16)[:, :6].t()) == (16, C_)
    assert g.operand_layout(torch.empty(1, 5)) == (5, R)
    assert g.operand_layout(torch.empty(5, 1)) == (1, R)
    with pytest.raises(ValueError):
        g.operand_layout(torch.empty(6, 10)[:, ::2])
    with pytest.raises(ValueError):
        g.operand_layout(torch.empty(2, 3, 4))


SCHED_CHECK = r"""
#include "common.hpp"
#include <cstdio>
#include <vector>
// For each grid: every workgroup id maps to a distinct in-range tile, and the ids one XCD
// receives (w % 8 equal) cover tiles that share few row/column panels.
int main() {
    const int shapes[][3] = {{16,16,4},{16,16,1},{1,1,1},{3,5,2},{8,43,4},{16,86,8},{33,17,4},
                             {1,64,1},{7,9,8},{32,32,4},{2,344,2},{16,16,0},{3,5,0}};
    for (auto& s : shapes) {
        const int tm_ = s[0], tn_ = s[1], gm = s[2];
        std::vector<int> seen(tm_ * tn_, 0);
        for (int w = 0; w < tm_ * tn_; ++w) {
            int a, b;
            gemm::tile_coords(w, tm_, tn_, gm, a, b);
            if (a < 0 || a >= tm_ || b < 0 || b >= tn_) { printf("range %d %d %d\n", tm_, tn_, w); return 1; }
            if (seen[a * tn_ + b]++) { printf("dup %d %d %d\n", tm_, tn_, w); return 1; }
        }
    }
    // 4096^2 output in 256^2 tiles, group 4: XCD x gets a 4 x 8 block of tiles
    for (int x = 0; x < 8; ++x) {
        int rmin = 99, rmax = -1, cmin = 99, cmax = -1;
        for (int w = x; w < 256; w += 8) {
            int a, b;
            gemm::tile_coords(w, 16, 16, 4, a, b);
            rmin = a < rmin ? a : rmin; rmax = a > rmax ? a : rmax;
            cmin = b < cmin ? b : cmin; cmax = b > cmax ? b : cmax;
        }
        if (rmax - rmin != 3 || cmax - cmin != 7) { printf("xcd %d block %d x %d\n", x, rmax-rmin+1, cmax-cmin+1); return 1; }
    }
    // group_m 0: both remaps off, tiles in row-major order of the workgroup id
    for (int w = 0; w < 15; ++w) {
        int a, b;
        gemm::tile_coords(w, 3, 5, 0, a, b);
        if (a != w / 5 || b != w % 5) { printf("plain order %d\n", w); return 1; }
    }
    // strided batches: a bijection onto (entry, tile) for several tile grids (below and above 16
    // tiles per entry), entry counts and
    // group heights
    const int bshapes[][3] = {{8, 1, 32}, {8, 8, 32}, {3, 5, 7}, {1, 1, 9}, {16, 16, 3}, {5, 2, 17}};
    for (const auto& sh : bshapes)
        for (int gm : {0, 1, 2, 4}) {
            const int tm_ = sh[0], tn_ = sh[1], nz = sh[2];
            std::vector<int> seen(tm_ * tn_ * nz, 0);
            for (int z = 0; z < nz; ++z)
                for (int x = 0; x < tm_ * tn_; ++x) {
                    int e, a, b;
                    gemm::batch_tile_coords(x, z, nz, tm_, tn_, gm, e, a, b);
                    if (e < 0 || e >= nz || a < 0 || a >= tm_ || b < 0 || b >= tn_) { printf("batch range\n"); return 1; }
                    if (seen[(e * tm_ + a) * tn_ + b]++) { printf("batch dup %d %d %d\n", tm_, tn_, nz); return 1; }
                }
        }
    // attention P.V: 8 tiles per entry, 32 entries; the workgroups of XCD x (dispatch ids
    // x, x + 8, ...) take entries 4x .. 4x+3 whole
    for (int x = 0; x < 8; ++x)
        for (int w = x; w < 256; w += 8) {
            int e, a, b;
            gemm::batch_tile_coords(w % 8, w / 8, 32, 8, 1, 8, e, a, b);
            if (e / 4 != x) { printf("batch xcd %d entry %d\n", x, e); return 1; }
        }
    printf("ok\n");
    return 0;
}
"""


def test_tile_scheduler_is_a_bijection_with_xcd_blocks():
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "sched.hip")
        exe = os.path.join(d, "sched")
        open(src, "w").write(SCHED_CHECK)
        subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O1",
                        f"-I{os.path.join(ROOT, 'gemm_f32_amd', 'csrc')}", src, "-o", exe],
                       check=True, capture_output=True)
        r = subprocess.run([exe], capture_output=True, text=True)
        assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout


# --- the default kernel choice, without a device (gemm_plan) -----------------------------
KNOWN_KERNELS = {"f32_dma256x256", "f32_dma128x128", "f32_mfma128x128", "f32_mfma64x64",
                 "f32_skinny16", "f32_skinny64", "f32_skinny32_halves", "f32_skinny32", "bf16_skinny32", "bf16_dma256x256", "bf16_dma256x128",
                 "bf16_mfma256x128", "bf16_mfma128x128", "bf16_mfma64x64",
                 "bf16_skinny16", "bf16_skinny64", "zero_c", "none"}


@pytest.mark.parametrize("dtype,shape,orders,expected", [
    ("f32", (4096, 4096, 4096), (R, R, R), ("f32_dma256x256", 4096, 4096)),
    ("bf16", (4096, 4096, 4096), (R, C_, R), ("bf16_dma256x256", 4096, 4096)),
    # one round of 256^2 tiles, the last row of tiles overhanging M; column 4096 as a strip
    ("f32", (4095, 4097, 1023), (R, R, R), ("f32_dma256x256", 4095, 4096)),
    ("bf16", (4095, 4097, 1023), (R, C_, R), ("bf16_dma256x256", 4095, 4096)),
    # 8 x 32 tiles of 256^2 fill one round; columns 8192 .. 11007 as a strip
    ("bf16", (2048, 11008, 4096), (R, C_, R), ("bf16_dma256x256", 2048, 8192)),
    ("bf16", (2048, 4096, 4096), (R, C_, R), ("bf16_dma256x128", 2048, 4096)),
    ("bf16", (2048, 4096, 11008), (R, C_, R), ("bf16_dma256x128", 2048, 4096)),
    # few FP32 rows with row-major B: two K halves of 32-column blocks (as many workgroups as
    # 16-column blocks) where K is long, N and ldb even; else 16-column blocks over the whole of K
    ("f32", (16, 4096, 4096), (R, R, R), ("f32_skinny32_halves", 16, 4096)),
    ("f32", (4096, 16, 4096), (C_, C_, C_), ("f32_skinny32_halves", 16, 4096)),
    ("f32", (16, 2048, 8192), (R, R, R), ("f32_skinny32_halves", 16, 2048)),
    ("f32", (16, 4096, 2048), (R, R, R), ("f32_skinny16", 16, 4096)),
    ("f32", (16, 4095, 4096), (R, R, R), ("f32_skinny16", 16, 4095)),
    ("f32", (17, 4096, 4096), (R, R, R), ("f32_skinny16", 17, 4096)),
    ("f32", (16, 4096, 4096), (R, C_, R), ("f32_skinny16", 16, 4096)),
    # 16-column blocks would take more than one round: 32-column blocks over the whole of K
    ("f32", (16, 8192, 4096), (R, R, R), ("f32_skinny32", 16, 8192)),
    ("f32", (16, 5120, 512), (R, R, R), ("f32_skinny32", 16, 5120)),
    ("f32", (16, 8192, 511), (R, R, R), ("f32_skinny16", 16, 8192)),
    ("f32", (16, 8191, 4096), (R, R, R), ("f32_skinny16", 16, 8191)),
    ("f32", (16, 8191, 4096), (R, C_, R), ("f32_skinny32", 16, 8191)),
    ("bf16", (16, 8192, 1024), (R, C_, R), ("bf16_skinny32", 16, 8192)),
    ("bf16", (16, 4096, 4096), (R, C_, R), ("bf16_skinny16", 16, 4096)),
    # 16-bit inputs: 64 x 64 register-staged tiles where the small-problem kernel's 64-column
    # blocks would leave CUs idle but the tiles fill at least half of them in one round (K <= 2048);
    # the small-problem kernel where its 64-column blocks fill the CUs, for longer K, few rows or
    # fewer tiles
    ("bf16", (1000, 1000, 1000), (R, C_, R), ("bf16_skinny64", 1000, 1000)),
    ("bf16", (768, 768, 768), (R, C_, R), ("bf16_mfma64x64", 768, 768)),
    ("bf16", (800, 1200, 1000), (R, C_, R), ("bf16_mfma64x64", 800, 1200)),
    ("bf16", (768, 768, 4000), (R, C_, R), ("bf16_skinny16", 768, 768)),
    ("bf16", (512, 512, 1024), (R, C_, R), ("bf16_skinny16", 512, 512)),
    ("f32", (1000, 1000, 1000), (R, R, R), ("f32_skinny64", 1000, 1000)),
    # column-major A: no overhang along M, so the core stops at the last whole row of tiles
    # (a planner bug once let a one-round candidate overhang there; the launch refused it)
    ("f32", (1055, 4096, 512), (C_, R, R), ("f32_dma128x128", 1024, 4096)),
    ("f32", (2054, 2048, 512), (C_, R, R), ("f32_dma128x128", 2048, 2048)),
    # column-major C: the library computes C^T (N x M)
    ("bf16", (4097, 4095, 1023), (R, C_, C_), ("bf16_dma256x256", 4095, 4096)),
    # row-major B with N % 8 == 0 takes the direct-copy tiles (transposing LDS reads of B), also
    # through the column-major-C swap from all column-major; N % 8 != 0 the register-staged ones
    ("bf16", (4096, 4096, 4096), (R, R, R), ("bf16_dma256x256", 4096, 4096)),
    ("bf16", (4096, 4096, 4096), (C_, C_, C_), ("bf16_dma256x256", 4096, 4096)),
    ("bf16", (2048, 4096, 4096), (R, R, R), ("bf16_dma256x128", 2048, 4096)),
    ("bf16", (4096, 4100, 4096), (R, R, R), ("bf16_mfma128x128", 4096, 4100)),
    ("f32", (64, 64, 0), (R, R, R), ("zero_c", 64, 64)),
    ("f32", (0, 64, 8), (R, R, R), ("none", 0, 0)),
], ids=lambda v: str(v))
def test_plan_of_known_shapes(dtype, shape, orders, expected):
    assert g.gemm_plan(dtype, *shape, *orders) == expected


def test_plan_rejects_invalid_arguments():
    for kw in (dict(cus=0), dict(M=-1), dict(K=2**31)):
        a = dict(dtype="f32", M=8, N=8, K=8, order_a=R, order_b=R, order_c=R, cus=256)
        a.update(kw)
        with pytest.raises(g.GemmError) as e:
            g.gemm_plan(**a)
        assert e.value.status == INVALID
    with pytest.raises(g.GemmError):
        g.gemm_plan("f32", 8, 8, 8, 2, R, R)


def test_plan_invariants_on_random_shapes():
    """Over random shapes and orders: the core lies inside C; kernels that take any shape
    cover all of it; the FP32 direct-copy core ends on whole tiles except along the edge of a
    k-contiguous operand (row-major A: M; column-major B: N), where its tiles may overhang; the
    16-bit direct-copy kernel runs on row-major A with column-major B, or row-major B and N a
    multiple of 8."""
    import numpy as np
    rng = np.random.default_rng(2024)
    for _ in range(400):
        dtype = "bf16" if rng.random() < 0.5 else "f32"
        M, N = (int(x) for x in rng.integers(1, 9000, 2))
        K = int(rng.integers(1, 5000))
        oa, ob, oc = (int(x) for x in rng.integers(0, 2, 3))
        if dtype == "bf16" and rng.random() < 0.7:
            oa, ob = R, C_                      # mostly the direct-copy kernel's layout
        kernel, rows, cols = g.gemm_plan(dtype, M, N, K, oa, ob, oc)
        assert kernel in KNOWN_KERNELS, kernel
        # the orientation the library computes in
        Mn, Nn, an, bn = (M, N, oa, ob) if oc == R else (N, M, 1 - ob, 1 - oa)
        assert 0 < rows <= Mn and 0 < cols <= Nn, (kernel, M, N, rows, cols)
        if "skinny" in kernel or "mfma" in kernel:
            assert (rows, cols) == (Mn, Nn), (kernel, M, N, oc, rows, cols)
        if kernel.startswith("f32_dma"):
            t = 256 if kernel == "f32_dma256x256" else 128
            assert rows % t == 0 or (an == R and rows == Mn), (kernel, M, N, oa, ob, oc, rows)
            assert cols % t == 0 or (bn == C_ and cols == Nn), (kernel, M, N, oa, ob, oc, cols)
        if kernel.startswith("bf16_dma"):
            assert an == R and (bn == C_ or Nn % 8 == 0), (kernel, M, N, oa, ob, oc)


@pytest.mark.parametrize("dtype,shape,orders,expected", [
    # 64 blocks of 16 x 16 leave most of 256 CUs idle: 16 slabs of 64 columns x 16 K slices
    ("f32", (16, 1024, 16384), (R, R, R), 16 * 16 * 1024 * 4),
    ("bf16", (16, 1024, 16384), (R, C_, R), 16 * 16 * 1024 * 4),
    # its own 256 blocks fill the chip: no split
    ("f32", (16, 4096, 4096), (R, R, R), 0),
    ("f32", (4096, 4096, 4096), (R, R, R), 0),
    # K too short for even two slices of one batch per wavefront
    ("f32", (16, 1024, 500), (R, R, R), 0),
    # blocks of 16 columns that need two rounds: one round of 64-column blocks in 2 K slices; one
    # exact round of them (16 x 4096 x 4096) stays unsplit
    ("f32", (16, 8192, 8192), (R, R, R), 2 * 16 * 8192 * 4),
    ("f32", (32, 8192, 4096), (R, R, R), 2 * 32 * 8192 * 4),
    ("f32", (16, 4096, 4096), (R, R, R), 0),
    ("bf16", (16, 4096, 4096), (R, C_, R), 0),
    # column-major C: C^T has the few rows
    ("f32", (1024, 16, 16384), (C_, C_, C_), 16 * 16 * 1024 * 4),
    # 16-bit inputs on 256 x 256 tiles that leave CUs idle: one GPU's column shard of 4096^3 in
    # 5 K slices, 2048^2 x 8192 in 4 (slices 1 .. S-1 as M x N FP32 slabs), FFN-down 2048 x 4096
    # x 11008 in 2 (128 tiles of 256^2 against one round of 256 x 128 tiles); none where the
    # tiles fill the chip or where the unsplit 256 x 128 kernel is estimated as fast
    ("bf16", (4096, 512, 4096), (R, C_, R), 4 * 4096 * 512 * 4),
    ("bf16", (2048, 2048, 8192), (R, C_, R), 3 * 2048 * 2048 * 4),
    ("bf16", (4096, 4096, 4096), (R, C_, R), 0),
    ("bf16", (2048, 4096, 4096), (R, C_, R), 0),
    ("bf16", (2048, 4096, 11008), (R, C_, R), 1 * 2048 * 4096 * 4),
    # 16-bit 1000^3: the small-problem kernel's 64-column blocks fill the CUs (no split); 768^3
    # runs on 64 x 64 register-staged tiles, which never split
    ("bf16", (1000, 1000, 1000), (R, C_, R), 0),
    ("bf16", (768, 768, 768), (R, C_, R), 0),
    # FP32: whole 256 x 256 tiles split into one round's worth of slices of at least 512 where the
    # time model prices that below the default plan: the shard's 32 tiles in 8 slices, 2048^2 in 4;
    # not 4096 x 768 x 2048 (short slices), not ragged M, not tiles that fill the chip
    ("f32", (4096, 512, 4096), (R, R, R), 7 * 4096 * 512 * 4),
    ("f32", (4096, 512, 8000), (C_, C_, R), 7 * 4096 * 512 * 4),
    ("f32", (2048, 2048, 4096), (R, R, R), 3 * 2048 * 2048 * 4),
    ("f32", (4096, 768, 2048), (C_, R, R), 0),
    ("f32", (4096, 4096, 4096), (R, C_, R), 0),
    ("f32", (4100, 512, 4096), (R, R, R), 0),
], ids=lambda v: str(v))
def test_split_k_workspace_of_known_shapes(dtype, shape, orders, expected):
    assert g.gemm_plan(dtype, *shape, *orders, with_workspace=True)[3] == expected


@pytest.mark.parametrize("shape,expected", [
    ((4096, 4096, 4096), ("f16_dma256x256", 4096, 4096)),
    ((2048, 11008, 4096), ("f16_dma256x256", 2048, 8192)),
    ((16, 4096, 4096), ("f16_skinny16", 16, 4096)),
], ids=str)
def test_f16_plans_follow_bf16(shape, expected):
    """fp16 inputs take the same kernels and plans as bf16, under their own names."""
    assert g.gemm_plan("f16", *shape, R, C_, R) == expected
    bf = g.gemm_plan("bf16", *shape, R, C_, R)
    assert bf[1:] == expected[1:] and bf[0] == expected[0].replace("f16_", "bf16_")


# --- strided batched calls: validation happens before any device call --------------------
BATCHED = {"f32": g.gemm_f32_strided_batched, "bf16": g.gemm_bf16_f32acc_strided_batched,
           "f16": g.gemm_f16_f32acc_strided_batched}


def bargs(batch=3, M=8, N=8, K=8, A=FAKE, lda=8, sa=64, oa=R, B=FAKE, ldb=8, sb=64, ob=R, C=FAKE, ldc=8,
          sc=64, oc=R):
    return (batch, M, N, K, A, lda, sa, oa, B, ldb, sb, ob, C, ldc, sc, oc, 0)


@pytest.mark.parametrize("bad", [
    dict(batch=-1), dict(sa=-1), dict(sb=-8), dict(sc=-64), dict(M=-1), dict(ldc=7), dict(A=0),
    dict(C=FAKE + 2), dict(oc=3),
    dict(sc=63),                                   # stacked entries one element too close
    dict(sc=0),                                    # every entry on the same C
    dict(ldc=24, sc=8),                            # side by side needs 3 x 8 <= 24 ... and 8 >= N
    dict(ldc=23, sc=8, N=8),                       # third entry would run past ldc: overlaps row 1
    dict(ldc=24, sc=7),                            # side by side closer than N
    dict(oc=C_, M=4, N=8, ldc=4, sc=31),           # column-major C: entry span (8-1)*4 + 4 = 32
    dict(batch=2**40, sa=2**40),                   # entry offsets beyond int64 bytes
], ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_batched_invalid_arguments(dtype, bad):
    if bad == dict(ldc=24, sc=8):
        pytest.skip("3 entries of 8 columns fill ldc 24 exactly: a valid layout")
    assert _status(BATCHED[dtype], *bargs(**bad)) == INVALID


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", [dict(batch=0), dict(M=0), dict(N=0)])
def test_batched_empty_is_ok_without_launch(dtype, shape):
    assert _status(BATCHED[dtype], *bargs(**shape)) == g.Status.OK
    assert g.gemm_last_kernel() == "none"


@pytest.mark.skipif(gpu_available(), reason="checks the no-GPU path")
@pytest.mark.parametrize("layout", [
    dict(sc=64),                          # stacked, dense
    dict(sc=100),                         # stacked with a gap
    dict(ldc=24, sc=8),                   # side by side: [rows, entries, cols]
    dict(ldc=32, sc=10),                  # side by side with gaps
    dict(sa=0, sb=0),                     # one A and one B for every entry
    dict(oc=C_, M=4, N=8, ldc=4, sc=32),  # column-major C stacked
    dict(batch=1, sc=0),                  # one entry: no stride matters
], ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_batched_valid_layouts_reach_the_device_check(layout):
    assert _status(BATCHED["f32"], *bargs(**layout)) == g.Status.ERR_UNSUPPORTED_DEVICE


# --- fused epilogue: argument checks before any device call -------------------------------
FUSED = {"bf16": g.gemm_bf16_f32acc_fused, "f16": g.gemm_f16_f32acc_fused, "f32": g.gemm_f32_fused}


def fargs(M=8, N=8, K=64, A=FAKE, lda=64, oa=R, B=FAKE, ldb=64, ob=C_, C=FAKE, ldc=8, oc=R):
    return (M, N, K, A, lda, oa, B, ldb, ob, C, ldc, oc)


@pytest.mark.parametrize("bad", [
    dict(call=dict(N=6, ldc=6, ob=R, ldb=6)),     # row-major B needs N % 8 == 0 (FP32: R,C only)
    dict(call=dict(oa=C_, lda=8)),
    dict(call=dict(K=32, lda=32, ldb=32)),        # 0 < K < 64
    dict(call=dict(C=FAKE + 2)),                  # FP32 output needs 4-byte alignment
    dict(call=dict(C=FAKE + 1), epi=dict(out_type=g.Out.BF16)),
    dict(epi=dict(activation=3)), dict(epi=dict(out_type=2)), dict(epi=dict(bias=FAKE + 2)),
    dict(call=dict(M=-1)), dict(call=dict(ldc=7)),
], ids=lambda d: ",".join(f"{k}={v}" for k, v in {**d.get("call", {}), **d.get("epi", {})}.items()))
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_fused_invalid_arguments(dtype, bad):
    if dtype == "f32" and bad.get("call", {}).get("K") == 32:
        pytest.skip("K = 32 is one whole FP32 k-tile: valid for FP32 inputs")
    assert _status(FUSED[dtype], *fargs(**bad.get("call", {})), **bad.get("epi", {})) == INVALID


@pytest.mark.parametrize("call", [dict(K=31, lda=31, ldb=31), dict(K=16, lda=16, ldb=16), dict(A=FAKE + 2),
                                  dict(oa=C_, lda=8)])
def test_f32_fused_invalid_arguments(call):
    """FP32 inputs: K >= 32 (one k-tile of the FP32 direct-copy kernel), 4-byte aligned operands."""
    assert _status(FUSED["f32"], *fargs(**call)) == INVALID


@pytest.mark.skipif(gpu_available(), reason="checks the no-GPU path")
def test_f32_fused_valid_call_reaches_the_device_check():
    assert _status(FUSED["f32"], *fargs(K=32, lda=32, ldb=32), activation=g.Act.RELU,
                   bias=FAKE) == g.Status.ERR_UNSUPPORTED_DEVICE


def test_fused_null_epilogue_rejected():
    rc = g.lib_handle().gemm_bf16_f32acc_fused(*fargs(), None, None)
    assert rc == INVALID


@pytest.mark.skipif(gpu_available(), reason="checks the no-GPU path")
@pytest.mark.parametrize("call", [dict(), dict(oc=C_), dict(K=0), dict(C=FAKE + 2, ldc=8), dict(ob=R, ldb=8)])
def test_fused_valid_calls_reach_the_device_check(call):
    out = g.Out.BF16 if call.get("C") == FAKE + 2 else g.Out.F32
    assert _status(FUSED["bf16"], *fargs(**call), activation=g.Act.GELU, bias=FAKE,
                   out_type=out) == g.Status.ERR_UNSUPPORTED_DEVICE
