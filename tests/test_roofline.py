"""The cost model reproduces the numbers the pages print (CPU only)."""
import math
import os

import pytest

from gemm_f32_amd import roofline as rl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# Device figures behind the "GEMM, step by step" model table.  Printed on the pages:
# A100 FP32 roof 19.5 TFLOP/s and a tensor roof 16x higher; H100 3.35 TB/s HBM and
# 67 TFLOP/s FP32.  Not printed (datasheet readings): A100 HBM 1.555 TB/s; shared memory
# = SMs x 128 B/clk x boost clock (A100 108 x 1.41 GHz, H100 132 x 1.98 GHz).
A100_FP32 = rl.Device("A100", 19.5e12, 1.555e12, 108 * 128 * 1.41e9)
A100_TC = rl.Device("A100-tc", 16 * 19.5e12, 1.555e12, 108 * 128 * 1.41e9)
H100_FP32 = rl.Device("H100", 67e12, 3.35e12, 132 * 128 * 1.98e9)
H100_TC = rl.Device("H100-tc", 989e12, 3.35e12, 132 * 128 * 1.98e9)


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [l.split() for l in f if l.strip() and not l.startswith("#")]


def _sig3(x, y):
    """x printed to 3 significant digits equals y."""
    return float(f"{x:.3g}") == float(f"{y:.3g}")


N = 4096
MODELS = {
    "naive": (rl.kernel_model(N, N, N, 1, 1, 1, eb=4, staged=False), A100_FP32, H100_FP32, True),
    "smem_tiles_32": (rl.kernel_model(N, N, N, 32, 32, 32, 1, 1, eb=4), A100_FP32, H100_FP32, True),
    "register_blocking_128": (rl.kernel_model(N, N, N, 128, 128, 8, 8, 8, eb=4), A100_FP32, H100_FP32, True),
    # the tensor-core row is priced on arithmetic and HBM only ("HBM (no L2 reuse)")
    "tensor_cores_bf16_128": (rl.kernel_model(N, N, N, 128, 128, 32, 8, 8, eb=2), A100_TC, H100_TC, False),
}


@pytest.mark.parametrize("row", _rows("p1_model_table.txt"), ids=lambda r: r[0])
def test_p1_model_table(row):
    name, fpb, t_a100, t_h100 = row[0], float(row[1]), float(row[2]), float(row[3])
    model, a100, h100, smem = MODELS[name]
    assert _sig3(model.intensity, fpb), (name, model.intensity)
    assert _sig3(model.time(a100, smem), t_a100), (name, model.time(a100, smem))
    assert _sig3(model.time(h100, smem), t_h100), (name, model.time(h100, smem))


@pytest.mark.parametrize("row", _rows("p5_traffic_table.txt"), ids=lambda r: "T" + r[0])
def test_p5_traffic_table(row):
    T, intensity, gb = int(row[0]), float(row[1]), float(row[2])
    if T == 0:
        m = rl.kernel_model(N, N, N, 1, 1, 1, eb=4, staged=False, c_bytes=0)
    else:
        m = rl.kernel_model(N, N, N, T, T, T, 1, 1, eb=4, c_bytes=0)
    assert math.isclose(m.intensity, intensity, rel_tol=1e-12)
    assert round(m.glob_bytes / 1e9, 1) == gb


def test_intensity_formulas():
    # "GEMM, step by step", Maths: b/4 for square FP32 blocks, b/2 for BF16; 1/4 and 2
    # flop/byte of shared memory for a 1x1 and an 8x8 patch.
    assert rl.global_intensity(128, 128, 4) == 32.0
    assert rl.global_intensity(128, 128, 2) == 64.0
    assert rl.smem_intensity(1, 1) == 0.25
    assert rl.smem_intensity(8, 8) == 2.0
    # bk cancels out of the block's global intensity
    a = rl.kernel_model(1024, 1024, 1024, 64, 64, 8, c_bytes=0).intensity
    b = rl.kernel_model(1024, 1024, 1024, 64, 64, 32, c_bytes=0).intensity
    assert math.isclose(a, b) and math.isclose(a, rl.global_intensity(64, 64, 4))


def test_flops_and_compulsory_bytes():
    assert rl.gemm_flops(4096, 4096, 4096) == 2 * 4096 ** 3
    # "How a Matrix Multiply Runs on a GPU": 4096^2 BF16 operands, ~1.37e11 flops over
    # at least 100 MB, about 1365 flop/byte (all three matrices at 2 bytes)
    f = rl.gemm_flops(4096, 4096, 4096)
    assert round(f / 1e11, 2) == 1.37
    by = rl.compulsory_bytes(4096, 4096, 4096, 2, 2)
    assert by >= 100e6 and round(f / by) == 1365
    # MI355X roofs
    assert math.isclose(rl.MI355X_BF16_DENSE_FLOPS, 256 * 4096 * 2.4e9, rel_tol=1e-4)
    assert math.isclose(rl.MI355X_FP32_FLOPS, 256 * 256 * 2.4e9, rel_tol=1e-3)
