"""Shader clock and cycle budget of the two 4096^3 kernels, read by the kernels themselves.

    python -m gemm_f32_amd.clockprobe build            # instrumented copy: libgemm_probe.so
    python -m gemm_f32_amd.clockprobe run [--reps N]   # bench.py's default step through it

The matrix cores of an MI355X run at whatever clock the board's power limit allows under the
current load, so a kernel's time alone does not say how many cycles it spent nor how busy its
matrix instructions kept the SIMDs.  `build` makes a copy of the two direct-copy kernel sources
(bf16_dma.hip, f32_dma.hip) in which the plain whole-tile kernels record, per wavefront, the
shader clock counter (s_memtime) and the 100 MHz constant clock (s_memrealtime) at three points --
entry, the end of the k-loop, and after the epilogue's stores are issued -- into a device array.
Nothing else in the kernels changes.  The copy is compiled with the library's flags and linked
with the library's other objects (gemm_f32_amd/_build/*.o, from `python -m gemm_f32_amd.build`)
into gemm_f32_amd/libgemm_probe.so.  `run` executes the default benchmark step (FP32 4096^3 GEMM,
then BF16 4096^3 GEMM, inputs rotating over several sets as in bench.py) through that library and
prints per leg, as medians over wavefronts and launches:

  * the clock: shader cycles over constant-clock time between entry and end;
  * entry -> end of the k-loop in cycles, and per k-tile, against the matrix instructions' own
    cycles per k-tile on one SIMD (BF16: 64 instructions of 32 cycles on the SIMD's one
    wavefront; FP32: 2 x 256 instructions of 32 cycles on its two);
  * the epilogue (end of k-loop -> stores issued) in cycles and microseconds;
  * the spread of the wavefronts' start and end times over the launch.

With --fp8 the step also runs the E4M3 4096^3 GEMM (same direct-copy kernel, 8-bit build).

This is measurement tooling; the library itself is not changed by it.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROBE = os.path.join(PKG, "_build", "probe")
LIB = os.path.join(PKG, "libgemm_probe.so")

_ARRAY = "__device__ unsigned long long g_clk_{tag}[{n}][6];\n"


def _stamp(var: str) -> str:
    return f"const uint64_t {var}_t = __builtin_amdgcn_s_memtime(), {var}_rt = __builtin_amdgcn_s_memrealtime();\n"


def _record(tag: str, n: int, cond: str, waves: str) -> str:
    return (f"    if constexpr ({cond}) {{\n"
            f"        const uint64_t P2_t = __builtin_amdgcn_s_memtime(), P2_rt = __builtin_amdgcn_s_memrealtime();\n"
            f"        const unsigned idx = blockIdx.x * ({waves}) + (threadIdx.x >> 6);\n"
            f"        if ((threadIdx.x & 63) == 0 && idx < {n}) {{\n"
            f"            volatile unsigned long long* o = g_clk_{tag}[idx];\n"
            f"            o[0] = P0_rt; o[1] = P1_rt; o[2] = P2_rt; o[3] = P0_t; o[4] = P1_t; o[5] = P2_t;\n"
            f"        }}\n    }}\n")


def _replace_once(text: str, old: str, new: str, what: str) -> str:
    n = text.count(old)
    if n < 1:
        raise RuntimeError(f"clock probe: anchor for {what} not found; the kernel source changed")
    i = text.index(old)
    return text[:i] + new + text[i + len(old):]


def instrument_bf16(text: str) -> str:
    """bf16_dma.hip with timestamps in the plain ring kernel, 16- or 8-bit inputs (1024 wavefronts
    at 4096^2; the two builds never run at the same time, so they share the array)."""
    t = _replace_once(text, "namespace gemm {\nnamespace {\n",
                      _ARRAY.format(tag="bf16", n=1024) + "namespace gemm {\nnamespace {\n", "namespace")
    t = _replace_once(t, "    __shared__ __align__(16) unsigned char smem[C::LDS];\n",
                      "    __shared__ __align__(16) unsigned char smem[C::LDS];\n    " + _stamp("P0"), "kernel entry")
    t = _replace_once(t, "    // ---- epilogue: stores past M or N are skipped ----\n",
                      "    " + _stamp("P1") + "    // ---- epilogue: stores past M or N are skipped ----\n", "k-loop end")
    t = _replace_once(t, "\n}\n\n// One launch of configuration C",
                      "\n" + _record("bf16", 1024, "MODE == kPlain && C::RING", "C::NW")
                      + "}\n\n// One launch of configuration C", "kernel end")
    return t + ('\nextern "C" int gemm_probe_read_bf16(void* dst) {\n'
                '    return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(g_clk_bf16), sizeof(g_clk_bf16));\n}\n')


def instrument_f32(text: str) -> str:
    """f32_dma.hip with timestamps in the plain whole-tile FP32 kernel (2048 wavefronts at 4096^2)."""
    t = _replace_once(text, "namespace gemm {\nnamespace {\n",
                      _ARRAY.format(tag="f32", n=2048) + "namespace gemm {\nnamespace {\n", "namespace")
    entry = "    __shared__ __align__(16) unsigned char smem[S * C::STAGE];\n    if constexpr (SPLIT)"
    t = _replace_once(t, entry, "    __shared__ __align__(16) unsigned char smem[S * C::STAGE];\n    "
                      + _stamp("P0") + "    if constexpr (SPLIT)", "kernel entry")
    ep = "    // ---- epilogue: block (i, j), lane l, register v: block row 4 (l / 16) + v, block\n"
    t = _replace_once(t, ep, "    " + _stamp("P1") + ep, "k-loop end")
    t = _replace_once(t, "\n}\n\n// k_f32_dma_edge's plan",
                      "\n" + _record("f32", 2048, "!BATCH && !SPLIT && C::BM == 256", "C::NW")
                      + "}\n\n// k_f32_dma_edge's plan", "kernel end")
    return t + ('\nextern "C" int gemm_probe_read_f32(void* dst) {\n'
                '    return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(g_clk_f32), sizeof(g_clk_f32));\n}\n')


def build() -> str:
    from gemm_f32_amd import build as gb
    os.makedirs(PROBE, exist_ok=True)
    objs = []
    for src, fn in (("bf16_dma.hip", instrument_bf16), ("f32_dma.hip", instrument_f32)):
        text = fn(open(os.path.join(gb.CSRC, src)).read())
        path = os.path.join(PROBE, src)
        with open(path, "w") as f:
            f.write(text)
        obj = path.replace(".hip", ".o")
        cmd = [gb.hipcc(), *gb.FLAGS, *gb.EXTRA_FLAGS.get(src, []), "-c", path, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on the instrumented {src}:\n{r.stderr[-3000:]}")
        objs.append(obj)
    others = [os.path.join(gb.BUILD, s.replace(".hip", ".o")) for s in gb.SOURCES
              if s not in ("bf16_dma.hip", "f32_dma.hip")]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"build the library first (python -m gemm_f32_amd.build): missing {missing}")
    r = subprocess.run([gb.hipcc(), f"--offload-arch={gb.ARCH}", "-shared", "-fPIC", *others, *objs, "-o", LIB],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-3000:]}")
    return LIB


def run(reps: int, fp8: bool = False) -> None:
    import ctypes

    import numpy as np
    import torch

    if not os.path.exists(LIB):
        raise SystemExit(f"{LIB} is not built: python -m gemm_f32_amd.clockprobe build")
    lib = ctypes.CDLL(LIB)
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    args = [ci, i64, i64, i64, vp, i64, ci, vp, i64, ci, vp, i64, ci, vp]
    lib.gemm_f32_algo.argtypes = args
    lib.gemm_bf16_f32acc_algo.argtypes = args
    lib.gemm_probe_read_bf16.argtypes = [vp]
    lib.gemm_probe_read_f32.argtypes = [vp]
    lib.gemm_last_kernel.restype = ctypes.c_char_p
    lib.gemm_fp8_f32acc.argtypes = [i64, i64, i64, vp, i64, ci, ci, vp, i64, ci, ci, vp, i64, ci, vp]
    n = 4096
    fp8_sets = 17 if fp8 else 0          # more than 512 MB of 8-bit operands
    gen = torch.Generator(device="cuda").manual_seed(0)
    # inputs rotate over 5 (FP32) and 9 (BF16) independently drawn sets, as in bench.py, so that
    # operands come from HBM rather than the last-level cache
    fa = [torch.rand(n * n, device="cuda", generator=gen) * 2 - 1 for _ in range(5)]
    fb = [torch.rand(n * n, device="cuda", generator=gen) * 2 - 1 for _ in range(5)]
    ba = [(torch.rand(n * n, device="cuda", generator=gen) * 2 - 1).to(torch.bfloat16).view(torch.int16) for _ in range(9)]
    bb = [(torch.rand(n * n, device="cuda", generator=gen) * 2 - 1).to(torch.bfloat16).view(torch.int16) for _ in range(9)]
    c = torch.empty(n * n, device="cuda")
    # E4M3 operands: uniform [-1, 1] rounded by torch's conversion (the timing does not depend on
    # the rounding)
    qa = [(torch.rand(n * n, device="cuda", generator=gen) * 2 - 1).to(torch.float8_e4m3fn).view(torch.uint8)
          for _ in range(fp8_sets)]
    qb = [(torch.rand(n * n, device="cuda", generator=gen) * 2 - 1).to(torch.float8_e4m3fn).view(torch.uint8)
          for _ in range(fp8_sets)]
    st = torch.cuda.current_stream().cuda_stream
    legs = {
        "square4096_f32": (lambda s: lib.gemm_f32_algo(0, n, n, n, fa[s % 5].data_ptr(), n, 0, fb[s % 5].data_ptr(), n, 0,
                                                       c.data_ptr(), n, 0, st),
                           lib.gemm_probe_read_f32, 2048, 32, 2 * 256 * 32),
        "square4096_bf16": (lambda s: lib.gemm_bf16_f32acc_algo(0, n, n, n, ba[s % 9].data_ptr(), n, 0, bb[s % 9].data_ptr(),
                                                                n, 1, c.data_ptr(), n, 0, st),
                            lib.gemm_probe_read_bf16, 1024, 64, 64 * 32),
    }
    if fp8_sets:
        # 8-bit: a k-tile is 128 deep, 2 k-steps of 16 v_mfma_scale_f32_32x32x64_f8f6f4 of 64 cycles
        legs["square4096_e4m3"] = (
            lambda s: lib.gemm_fp8_f32acc(n, n, n, qa[s % fp8_sets].data_ptr(), n, 0, 0, qb[s % fp8_sets].data_ptr(), n,
                                          1, 0, c.data_ptr(), n, 0, st),
            lib.gemm_probe_read_bf16, 1024, 128, 32 * 64)
    stats = {k: [] for k in legs}
    kernels = {}
    warm = 3
    for s in range(warm + reps):
        for name, (go, read, waves, bk, ideal) in legs.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            rc = go(s)
            e1.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise SystemExit(f"{name}: status {rc}")
            kernels[name] = lib.gemm_last_kernel().decode()
            if s < warm:
                continue
            buf = np.zeros((waves, 6), dtype=np.uint64)
            if read(buf.ctypes.data) != 0:
                raise SystemExit("reading the probe array failed")
            b = buf.astype(np.float64)
            rt0, rt1, rt2, t0, t1, t2 = (b[:, i] for i in range(6))
            clk = (t2 - t0) / (rt2 - rt0) * 0.1                       # GHz (constant clock 100 MHz)
            stats[name].append(dict(
                event_us=e0.elapsed_time(e1) * 1e3, clock=np.median(clk), loop=np.median(t1 - t0),
                per_ktile=np.median(t1 - t0) / (n // bk), epi=np.median(t2 - t1),
                epi_us=np.median((rt2 - rt1) / 100.0), start_spread=(rt0.max() - rt0.min()) / 100.0,
                end_spread=(rt2.max() - rt2.min()) / 100.0, span=(rt2.max() - rt0.min()) / 100.0, ideal=ideal))
    print("| leg | kernel | launch µs (events) | shader clock GHz | entry -> k-loop end, cycles | per k-tile | "
          "matrix cycles per k-tile | loop busy | epilogue cycles (µs) | wavefronts' span µs | start / end spread µs |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for name, rows in stats.items():
        med = {k: float(np.median([r[k] for r in rows])) for k in rows[0]}
        print(f"| {name} | {kernels[name]} | {med['event_us']:.1f} | {med['clock']:.3f} | {med['loop']:.0f} | "
              f"{med['per_ktile']:.0f} | {med['ideal']:.0f} | {med['ideal'] / med['per_ktile']:.3f} | "
              f"{med['epi']:.0f} ({med['epi_us']:.1f}) | {med['span']:.1f} | {med['start_spread']:.2f} / "
              f"{med['end_spread']:.2f} |", flush=True)


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("build")
    r = sub.add_parser("run")
    r.add_argument("--reps", type=int, default=20)
    r.add_argument("--fp8", action="store_true", help="also the E4M3 4096^3 GEMM (gemm_fp8_f32acc)")
    a = ap.parse_args()
    if a.cmd == "build":
        print(build())
    else:
        sys.path.insert(0, ROOT)
        run(a.reps, a.fp8)


if __name__ == "__main__":
    main()
