"""What the GPU's memory delivers to the read and write patterns of the few-row products.

    python -m gemm_f32_amd.bwprobe build          # gemm_f32_amd/libbwprobe.so from bwprobe.hip
    python -m gemm_f32_amd.bwprobe run [--reps N]  # one table, launches timed with HIP events

The 16 x 4096 x 4096 products are bound by reading B once (64 MiB FP32, 32 MiB BF16).  The HBM
peak (8 TB/s) is not what a read of that size and shape can reach, so this tool times, on the
same rotating buffers, the patterns the products impose (bwprobe.hip describes each kernel):
a plain read of the whole buffer, a row-major B read 16 columns per workgroup (as one
16-column block of C needs it), the same with the small-problem FP32 kernel's 4-byte loads and
with its re-reads of A, 32 columns over half of K per workgroup (the library's two-halves mode
for few FP32 rows), one contiguous chunk per workgroup (a column-major B), and a plain write of a
64 MiB C.  Beside them it times the library's own calls on the same bytes (gemm_f32 R,R,R, whose
two-halves mode also zeroes C first, and gemm_bf16_f32acc R,C,R, 16 x 4096 x 4096).  Inputs
rotate over 9 buffers of 64 MiB, more than the 256 MB last-level cache holds, so every read
comes from HBM.  Run it under `rocprofv3 --kernel-trace --stats` for
kernel times without launch gaps.

This is measurement tooling; the library itself is not changed by it.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "bwprobe.hip")
LIB = os.path.join(PKG, "libbwprobe.so")

SETS = 9
N = 4096
K = 4096


def build() -> str:
    from gemm_f32_amd import build as gb
    cmd = [gb.hipcc(), *gb.FLAGS, "-shared", "-fPIC", SRC, "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"hipcc failed on bwprobe.hip:\n{r.stderr[-3000:]}")
    print(f"built {LIB}")
    return LIB


def _timed(fn, reps: int) -> float:
    """Mean microseconds per call of fn(i) over reps calls after 3 untimed ones, from HIP events
    recorded on the stream the calls launch on."""
    import torch
    for i in range(3):
        fn(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(reps):
        fn(i)
    t1.record()
    t1.synchronize()
    return t0.elapsed_time(t1) * 1e3 / reps


def run(reps: int) -> None:
    import ctypes
    import torch
    if not os.path.exists(LIB):
        raise SystemExit(f"{LIB} is missing: run `python -m gemm_f32_amd.bwprobe build` first")
    import gemm_f32_amd as g
    lib = ctypes.CDLL(LIB)
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.bwprobe_out_floats.restype = i64
    lib.bwprobe_plain.argtypes = [vp, i64, vp, vp]
    lib.bwprobe_slab16.argtypes = [vp, i64, ci, ci, ci, vp, vp]
    lib.bwprobe_skinny.argtypes = [vp, i64, ci, ci, ci, vp, i64, vp, vp]
    lib.bwprobe_w32h.argtypes = [vp, i64, ci, ci, ci, vp, i64, vp, vp]
    lib.bwprobe_chunk.argtypes = [vp, i64, vp, vp]
    lib.bwprobe_write.argtypes = [vp, i64, vp]

    torch.cuda.set_device(0)
    gen = torch.Generator(device="cuda").manual_seed(0)
    bs = [torch.rand(K * N, device="cuda", generator=gen) * 2 - 1 for _ in range(SETS)]
    as_ = [torch.rand(16 * K, device="cuda", generator=gen) * 2 - 1 for _ in range(SETS)]
    # BF16 operands: A 16 x K row-major, B K x N column-major (k-contiguous), as bit patterns
    b16 = [(torch.rand(K * N, device="cuda", generator=gen) * 2 - 1).to(torch.bfloat16) for _ in range(2 * SETS)]
    a16 = [(torch.rand(16 * K, device="cuda", generator=gen) * 2 - 1).to(torch.bfloat16) for _ in range(2 * SETS)]
    out = torch.empty(lib.bwprobe_out_floats(), device="cuda")
    c = torch.empty(16 * N, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    n = K * N

    def ok(rc: int, what: str) -> None:
        if rc != 0:
            raise RuntimeError(f"{what}: hipError {rc}")

    R, C_ = g.Order.ROW_MAJOR, g.Order.COL_MAJOR
    rows = [
        ("plain read, 1024 workgroups", "64 MiB", n * 4,
         lambda i: ok(lib.bwprobe_plain(bs[i % SETS].data_ptr(), n, out.data_ptr(), st), "plain")),
        ("plain read, 1024 workgroups", "32 MiB", n * 2,
         lambda i: ok(lib.bwprobe_plain(bs[i % SETS].data_ptr(), n // 2, out.data_ptr(), st), "plain")),
        ("row-major B, 16 columns per workgroup, 16-byte loads", "64 MiB", n * 4,
         lambda i: ok(lib.bwprobe_slab16(bs[i % SETS].data_ptr(), n, K, N, N, out.data_ptr(), st), "slab16")),
        ("the same slabs, small-problem kernel's 4-byte loads", "64 MiB", n * 4,
         lambda i: ok(lib.bwprobe_skinny(bs[i % SETS].data_ptr(), n, K, N, N, None, 0, out.data_ptr(), st), "skinny")),
        ("... and its reads of A (16 x 4096 FP32, from L2)", "64 MiB + A", n * 4,
         lambda i: ok(lib.bwprobe_skinny(bs[i % SETS].data_ptr(), n, K, N, N, as_[i % SETS].data_ptr(), 16 * K,
                                         out.data_ptr(), st), "skinny+A")),
        ("row-major B, 32 columns x half of K per workgroup", "64 MiB", n * 4,
         lambda i: ok(lib.bwprobe_w32h(bs[i % SETS].data_ptr(), n, K, N, N, None, 0, out.data_ptr(), st), "w32h")),
        ("... and the reads of A for that half", "64 MiB + A", n * 4,
         lambda i: ok(lib.bwprobe_w32h(bs[i % SETS].data_ptr(), n, K, N, N, as_[i % SETS].data_ptr(), 16 * K,
                                       out.data_ptr(), st), "w32h+A")),
        ("one contiguous chunk per workgroup, 256 workgroups", "32 MiB", n * 2,
         lambda i: ok(lib.bwprobe_chunk(bs[i % SETS].data_ptr(), n // 2, out.data_ptr(), st), "chunk")),
        ("plain write, 256 workgroups", "64 MiB", n * 4,
         lambda i: ok(lib.bwprobe_write(bs[i % SETS].data_ptr(), n, st), "write")),
        ("gemm_f32 16x4096x4096 R,R,R", "64 MiB + A + C", n * 4 + 2 * 16 * K * 4,
         lambda i: g.gemm_f32(16, N, K, as_[i % SETS].data_ptr(), K, R, bs[i % SETS].data_ptr(), N, R,
                              c.data_ptr(), N, R, st)),
        ("gemm_bf16_f32acc 16x4096x4096 R,C,R", "32 MiB + A + C", n * 2 + 16 * K * 2 + 16 * N * 4,
         lambda i: g.gemm_bf16_f32acc(16, N, K, a16[i % (2 * SETS)].data_ptr(), K, R, b16[i % (2 * SETS)].data_ptr(),
                                      K, C_, c.data_ptr(), N, R, st)),
    ]
    print("| pattern | bytes | µs per launch (events) | TB/s |")
    print("|---|---|---|---|")
    for name, what, nbytes, fn in rows:
        us = _timed(fn, reps)
        kern = f" (`{g.gemm_last_kernel()}`)" if name.startswith("gemm_") else ""
        print(f"| {name}{kern} | {what} | {us:.2f} | {nbytes / us / 1e6:.2f} |", flush=True)
    torch.cuda.synchronize()


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("build")
    r = sub.add_parser("run")
    r.add_argument("--reps", type=int, default=45)
    a = ap.parse_args(argv)
    if a.cmd == "build":
        build()
    else:
        run(a.reps)


if __name__ == "__main__":
    sys.path.insert(0, ROOT)
    main()
