"""Cost model of a tiled GEMM and the MI355X roofs it is measured against.

Host-side arithmetic only (no kernels).  It answers, for a kernel that computes
C = A.B in bm x bn blocks stepping through K in slices of bk, with each thread holding a
tm x tn patch of C:

* FLOPs = 2*M*N*K: one multiply and one add per term ("How a Matrix Multiply Runs on a
  GPU", section "The problem and the roofline"; "A06 - Tiled Matrix Multiply (GEMM)",
  "Pitfall 4 - Benchmarking artefacts").
* Global-memory intensity of a block, I = 2 / (e (1/bn + 1/bm)), independent of bk, and
  the shared-memory (LDS) intensity of a thread's patch, 2 tm tn / (4 (tm + tn))
  ("GEMM, step by step", section "Maths").
* Per-k-tile bytes of one block as the page's model counts them: a staged kernel moves
  e (bm bk + bk bn) bytes from global memory, writes that tile to shared memory and reads
  e bk (bm bn / (tm tn)) (tm + tn) bytes back; an unstaged kernel reads two operands per
  multiply-add, e bm bn 2 bk bytes ("GEMM, step by step", section "Code").
* Model time = the slowest of arithmetic, global traffic and shared-memory traffic.
  Each block writes its C tile once (4-byte values) when `c_bytes` is 4; the teaching
  module's traffic table leaves C out (`c_bytes=0`).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

# --- MI355X (gfx950) published figures; the roofs the measured kernels are priced on ---
MI355X_CUS = 256
MI355X_CLOCK_HZ = 2.4e9
MI355X_HBM_BYTES_PER_S = 8.0e12
MI355X_BF16_DENSE_FLOPS = 2516.6e12        # 256 CU x 4096 flop/clk x 2.4 GHz
MI355X_FP8_DENSE_FLOPS = 5033.2e12         # 256 CU x 8192 flop/clk x 2.4 GHz
MI355X_FP32_FLOPS = 157.3e12               # 256 CU x 256 flop/clk x 2.4 GHz (packed FMA / MFMA)
MI355X_FP32_VALU_UNPACKED_FLOPS = 78.6e12  # 256 CU x 4 SIMD x 16 lanes x 2 flop x 2.4 GHz


def gemm_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def compulsory_bytes(M: int, N: int, K: int, e_in: int, e_out: int = 4) -> int:
    """Every operand element crosses HBM once: A and B read, C written."""
    return e_in * (M * K + K * N) + e_out * M * N


def global_intensity(bm: int, bn: int, e: int) -> float:
    return 2.0 / (e * (1.0 / bn + 1.0 / bm))


def smem_intensity(tm: int, tn: int) -> float:
    return 2.0 * tm * tn / (4.0 * (tm + tn))


def ktile_bytes(bm: int, bn: int, bk: int, tm: int, tn: int, eb: int, staged: bool):
    """(global bytes, shared-memory bytes) one block moves for one k-tile."""
    if staged:
        tile = eb * (bm * bk + bk * bn)
        return tile, tile + eb * bk * (bm * bn // (tm * tn)) * (tm + tn)
    return eb * bm * bn * 2 * bk, 0


@dataclass(frozen=True)
class Device:
    name: str
    alu_flops: float        # roof of the arithmetic the kernel uses
    hbm_bytes_per_s: float
    smem_bytes_per_s: float


@dataclass(frozen=True)
class KernelModel:
    flops: float
    glob_bytes: float
    smem_bytes: float

    @property
    def intensity(self) -> float:
        return self.flops / self.glob_bytes

    def time(self, dev: Device, model_smem: bool = True) -> float:
        t = max(self.flops / dev.alu_flops, self.glob_bytes / dev.hbm_bytes_per_s)
        if model_smem and self.smem_bytes:
            t = max(t, self.smem_bytes / dev.smem_bytes_per_s)
        return t


def kernel_model(M: int, N: int, K: int, bm: int, bn: int, bk: int, tm: int = 1, tn: int = 1,
                 eb: int = 4, staged: bool = True, c_bytes: int = 4) -> KernelModel:
    blocks = math.ceil(M / bm) * math.ceil(N / bn)
    ktiles = math.ceil(K / bk)
    g, s = ktile_bytes(bm, bn, bk, tm, tn, eb, staged)
    return KernelModel(gemm_flops(M, N, K), blocks * (ktiles * g + c_bytes * bm * bn),
                       blocks * ktiles * s)


def mi355x_peak(dtype: str) -> float:
    # fp16 inputs: the same dense matrix-core peak as bf16 (2.5 PFLOP/s, published figures)
    # 8-bit inputs (every E4M3 / E5M2 pairing): the dense fp8 peak (5.0 PFLOP/s, published figures)
    if dtype in ("e4m3", "e5m2", "e4m3_e5m2", "e5m2_e4m3"):
        return MI355X_FP8_DENSE_FLOPS
    return {"bf16": MI355X_BF16_DENSE_FLOPS, "f16": MI355X_BF16_DENSE_FLOPS, "f32": MI355X_FP32_FLOPS}[dtype]
