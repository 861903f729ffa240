#!/usr/bin/env python3
"""Throughput of libgemm on one MI355X: GEMM TFLOP/s at 4096³ and fraction of peak.

One step is one pass of the whole hot path over resident synthetic inputs: an FP32 GEMM
(4096³, row-major A/B/C, uniform[-1, 1]) followed by a BF16-input, FP32-accumulate GEMM
(4096³, row-major A, column-major B, uniform[-1, 1] rounded to bf16), each through the
library's default kernel choice.  `value` is the FLOPs of the step (2MNK per GEMM, the
count the pages use) over the step time.  Per-kernel times come from HIP events recorded
between the launches on the launch stream; the roofline object prices the dominant
kernel against MI355X's published matrix-core peak for its dtype.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--algo NAME]

`--workload` picks another single workload from gemm_inputs.WORKLOADS (then one step is
that one GEMM, or one strided batched call for a batch workload such as attention's per-head
products); `--algo` forces a kernel (gemm_f32_amd.Algo name); `--epilogue NAME` calls the fused-epilogue entry point (bias, activation, bf16 output) for a
workload whose layout the fused calls take (row-major A with column-major B, or row-major A and B with N % 8 == 0); `--k K` replaces a single workload's K (a sweep over K separates a kernel's fixed
cost -- launch, first loads, the C write -- from its cost per k-tile); `--workspace` calls the
workspace entry points (gemm_f32_ws / gemm_bf16_f32acc_ws, split-K across workgroups where
the problem is too small to fill the device) with a workspace of the size the library asks
for, allocated before the timed region.  Each GEMM's inputs
rotate over enough independently drawn copies (`--sets`, default: at least 2 and more
than 512 MB of A and B together) that the 256 MB last-level cache cannot hold them across
steps.
The CPU baseline times the fp64 oracle on the host on a bounded sample of the same
problems (the first rows of C) and scales it to TFLOP/s.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s at 4096³ (FP32, BF16→FP32) and % of MI355X peak"
DEFAULT = "square4096"
DEFAULT_LEGS = ["square4096_f32", "square4096_bf16"]
# fused epilogues for --epilogue: (alpha, beta, bias, activation, bf16 output)
EPILOGUES = {"identity_f32": (1.0, 0.0, False, 0, False), "bias_gelu_bf16": (1.0, 0.0, True, 2, True),
             "beta_bias_relu_f32": (1.0, 1.0, True, 1, False)}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT)
    ap.add_argument("--algo", default="AUTO")
    ap.add_argument("--k", type=int, default=None,
                    help="replace the workload's K (same shape and recipe otherwise), for sweeps over K")
    ap.add_argument("--workspace", action="store_true",
                    help="use the workspace (split-K) entry points; AUTO only")
    ap.add_argument("--sets", type=int, default=0,
                    help="input copies per GEMM (0: enough for > 512 MB, at least 2)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target host time of the CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--epilogue", default=None, choices=sorted(EPILOGUES),
                    help="run the fused-epilogue entry point (16-bit inputs, row-major A, column-major B)")
    ap.add_argument("--tile-order", default="swizzled", choices=["swizzled", "rowmajor"],
                    help="rowmajor: the tile scheduler's XCD and group-M remaps off (GEMM_TILE_ORDER), to "
                         "measure what they buy")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain 256 MiB device-to-device copy instead (the reference "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters to bytes)")
    return ap.parse_args()


# sources that define each dominant kernel: its own file plus the shared headers (tile
# scheduler, buffer helpers) and the launch declarations
KERNEL_SOURCES = {
    "f32_dma": ("f32_dma.hip",),
    "bf16_dma": ("bf16_dma.hip", "mma16.hpp", "epilogue.hpp"),
    "f16_dma": ("bf16_dma.hip", "mma16.hpp", "epilogue.hpp"),
    "fp8_dma": ("bf16_dma.hip", "mma16.hpp", "epilogue.hpp"),
    "bf16_mfma": ("bf16_mfma.hip", "mma16.hpp"),
    "f32_skinny": ("skinny.hip", "mma16.hpp"),
    "bf16_skinny": ("skinny.hip", "mma16.hpp"),
}
SHARED_SOURCES = ("common.hpp", "launch.hpp")


def kernel_source_digest(kernel: str) -> str:
    """Hash of the sources a kernel is built from (the library's name for it, e.g.
    f32_dma256x256); counter-derived traffic is only reported for the sources it was
    measured on."""
    import hashlib
    family = next((k for k in KERNEL_SOURCES if kernel.startswith(k)), None)
    if family is None:
        return ""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gemm_f32_amd", "csrc")
    for name in sorted(KERNEL_SOURCES[family] + SHARED_SOURCES):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from profiles/traffic.json (FETCH_SIZE + WRITE_SIZE, scaled by
    the copy calibration), or None when absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(f"{kernel}@{workload}")
    digest = kernel_source_digest(kernel)
    if not rec or not digest or rec.get("source_digest") != digest:
        return None
    return rec["hbm_bytes_per_launch"]


def copy_calibration(args):
    import torch
    n = 256 * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "ms": round(ms, 4),
                      "GB/s": round(2 * n * 4 / (ms * 1e-3) / 1e9, 1)}), flush=True)


class Leg:
    """One GEMM of the step with its resident device buffers."""

    def __init__(self, name, algo, sets, workspace=False, epilogue=None, k=None):
        import dataclasses
        import torch
        import gemm_f32_amd as g
        import gemm_inputs as gi
        self.w = gi.WORKLOADS[name] if k is None else dataclasses.replace(gi.WORKLOADS[name], K=k)
        self.name = name
        self.algo = g.Algo[algo]
        self.problems = []
        self.A, self.B = [], []
        self.batched = self.w.batch > 1
        if self.batched and (algo != "AUTO" or workspace):
            raise SystemExit("a strided batch runs the default kernel choice without a workspace")
        fp8 = self.w.dtype in gi.FP8_DTYPES
        e = 4 if self.w.dtype == "f32" else 1 if fp8 else 2
        if fp8 and (algo != "AUTO" or workspace or self.batched or epilogue is not None):
            raise SystemExit("8-bit workloads run gemm_fp8_f32acc alone (one kernel family, no workspace)")
        if sets <= 0:
            per_set = e * self.w.batch * (self.w.M * self.w.K + self.w.K * self.w.N)
            sets = min(64, max(2, (512 * 2**20) // per_set + 1))
        self.sets = sets
        for s in range(sets):
            w = self.w
            p = gi.workload_problem(name, 1000 * s, K=k)
            self.problems.append(p)
            conv = (lambda b: b.view(np.int16)) if w.dtype in ("bf16", "f16") else (lambda b: b)
            self.A.append(torch.from_numpy(conv(p.A)).to("cuda"))
            self.B.append(torch.from_numpy(conv(p.B)).to("cuda"))
        p = self.problems[0]
        size = p.c_size() if self.batched else gi.c_buffer_size(p.M, p.N, p.ldc, p.order_c)
        self.C = torch.empty(size, dtype=torch.float32, device="cuda")
        if fp8:
            code = {"e4m3": g.Fp8.E4M3, "e5m2": g.Fp8.E5M2}
            fa, fb = code[gi.FP8_DTYPES[w.dtype][0]], code[gi.FP8_DTYPES[w.dtype][1]]
            self.fn = lambda algo, M, N, K, A, lda, oa, B, ldb, ob, C, ldc, oc, stream: g.gemm_fp8_f32acc(
                M, N, K, A, lda, oa, fa, B, ldb, ob, fb, C, ldc, oc, stream)
            self.fn_batched = None
        else:
            self.fn = {"f32": g.gemm_f32_algo, "bf16": g.gemm_bf16_f32acc_algo, "f16": g.gemm_f16_f32acc_algo}[w.dtype]
            self.fn_batched = {"f32": g.gemm_f32_strided_batched, "bf16": g.gemm_bf16_f32acc_strided_batched,
                               "f16": g.gemm_f16_f32acc_strided_batched}[w.dtype]
        self.flops = w.flops
        # compulsory HBM bytes: every input element read once, every output element written once
        self.bytes = w.batch * (e * (w.M * w.K + w.K * w.N) + 4 * w.M * w.N)
        self.kernel = None
        self.ws, self.ws_bytes = None, 0
        self.epi = None
        if epilogue is not None:
            if algo != "AUTO" or workspace or self.batched:
                raise SystemExit("--epilogue runs a fused entry point alone")
            alpha, beta, has_bias, act, out16 = EPILOGUES[epilogue]
            bias = torch.from_numpy(np.random.default_rng(1).uniform(-1, 1, w.N).astype(np.float32)).to("cuda")
            self.epi = (alpha, beta, bias if has_bias else None, act, 1 if out16 else 0)
            if out16:
                self.C = torch.zeros(size, dtype=torch.int16, device="cuda")
            else:
                self.C.zero_()
            self.fn_fused = {"bf16": g.gemm_bf16_f32acc_fused, "f16": g.gemm_f16_f32acc_fused,
                             "f32": g.gemm_f32_fused}[w.dtype]
        if workspace:
            if algo != "AUTO":
                raise SystemExit("--workspace runs the default kernel choice (--algo AUTO)")
            p0 = self.problems[0]
            self.ws_bytes = g.gemm_workspace_size(w.dtype, p0.M, p0.N, p0.K, p0.order_a, p0.order_b,
                                                  p0.order_c)
            self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device="cuda")
            self.fn_ws = {"f32": g.gemm_f32_ws, "bf16": g.gemm_bf16_f32acc_ws, "f16": g.gemm_f16_f32acc_ws}[w.dtype]

    def launch(self, s, stream):
        p = self.problems[s % len(self.problems)]
        if self.batched:
            self.fn_batched(p.batch, p.M, p.N, p.K, self.A[s % len(self.A)].data_ptr(), p.lda, p.sa, p.order_a,
                            self.B[s % len(self.B)].data_ptr(), p.ldb, p.sb, p.order_b, self.C.data_ptr(), p.ldc,
                            p.sc, p.order_c, stream)
            return
        if self.epi is not None:
            alpha, beta, bias, act, out = self.epi
            self.fn_fused(p.M, p.N, p.K, self.A[s % len(self.A)].data_ptr(), p.lda, p.order_a,
                          self.B[s % len(self.B)].data_ptr(), p.ldb, p.order_b, self.C.data_ptr(), p.ldc, p.order_c,
                          alpha=alpha, beta=beta, bias=bias.data_ptr() if bias is not None else 0, activation=act,
                          out_type=out, stream=stream)
            return
        if self.ws is not None:
            self.fn_ws(p.M, p.N, p.K, self.A[s % len(self.A)].data_ptr(), p.lda, p.order_a,
                       self.B[s % len(self.B)].data_ptr(), p.ldb, p.order_b, self.C.data_ptr(), p.ldc,
                       p.order_c, self.ws.data_ptr(), self.ws_bytes, stream)
            return
        self.fn(self.algo, p.M, p.N, p.K, self.A[s % len(self.A)].data_ptr(), p.lda, p.order_a,
                self.B[s % len(self.B)].data_ptr(), p.ldb, p.order_b, self.C.data_ptr(), p.ldc,
                p.order_c, stream)


def cpu_model() -> str:
    """The host CPU's model name (first "model name" line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(legs, target_s):
    """The oracle (as is) on the first R rows of each leg's problem, R sized to ~target_s."""
    import oracle
    threads = oracle.num_threads()

    import gemm_inputs as gi

    def run(rows):
        t0 = time.perf_counter()
        for leg in legs:
            p = leg.problems[0]
            a = p.A if p.order_a == 0 else None
            if a is None:                      # a column-major A: take the sub-matrix's rows
                sub = p.A_logical[:rows]
                a, lda = gi.lay_out(sub, 1)
            else:
                lda = p.lda
                a = p.A[: rows * p.lda]
            oracle.gemm(rows, p.N, p.K, a, lda, p.order_a, p.B, p.ldb, p.order_b, **gi.oracle_formats(p))
        return time.perf_counter() - t0

    probe = max(1, threads)
    t_probe = run(probe)
    rows = int(max(probe, min(min(l.w.M for l in legs), probe * target_s / max(t_probe, 1e-6))))
    rows = max(probe, (rows // probe) * probe)
    t = run(rows)
    flops = sum(2 * rows * l.w.N * l.w.K for l in legs)
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "nproc": os.cpu_count(), "cpu_model": cpu_model(), "seconds": round(t, 3),
            "sample": f"first {rows} rows of C for each of "
                      f"{', '.join(l.name + (' (entry 0)' if l.batched else '') for l in legs)} "
                      f"({flops / 2:.3e} multiply-adds, fp64 oracle, {threads} OpenMP threads)"}


TIMING = ("mean launch time from HIP events recorded before and after each launch on the "
          "launch stream, over the timed steps")


def leg_roofline(leg, info):
    """The roofline object of one leg's kernel: algorithmic work per launch (2MNK flops, or
    the compulsory bytes where those take longer at HBM's peak) over its mean launch time,
    against MI355X's published peak for the leg's dtype."""
    from gemm_f32_amd import roofline as rl
    peak = rl.mi355x_peak(leg.w.dtype)
    per = f" x {leg.w.batch} entries" if leg.batched else ""
    sec = info["ms"] * 1e-3
    if leg.bytes / rl.MI355X_HBM_BYTES_PER_S > leg.flops / peak:
        achieved = leg.bytes / sec
        return {"bound": "hbm", "kernel": info["kernel"], "achieved": round(achieved / 1e9, 1),
                "peak": rl.MI355X_HBM_BYTES_PER_S / 1e9, "unit": "GB/s",
                "frac": round(achieved / rl.MI355X_HBM_BYTES_PER_S, 4),
                "traffic": measured_traffic(info["kernel"], leg.name),
                "per_launch": f"e*(M*K + K*N) + 4*M*N{per} = {leg.bytes:.4e} B per launch ({leg.name})",
                "timing": TIMING}
    achieved = leg.flops / sec
    return {"bound": "mfma", "kernel": info["kernel"], "achieved": round(achieved / 1e12, 2),
            "peak": round(peak / 1e12, 1), "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(info["kernel"], leg.name),
            "per_launch": f"2*M*N*K{per} = {leg.flops:.4e} FLOP per launch ({leg.name})",
            "timing": TIMING}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args)
        return
    if args.tile_order == "rowmajor":
        os.environ["GEMM_TILE_ORDER"] = "rowmajor"     # read once, before the first call
    import torch
    import gemm_f32_amd as g
    from gemm_f32_amd import roofline as rl

    names = DEFAULT_LEGS if args.workload == DEFAULT else [args.workload]
    if args.k is not None and args.workload == DEFAULT:
        raise SystemExit("--k applies to a single --workload")
    legs = [Leg(n, args.algo, args.sets, args.workspace, args.epilogue, args.k) for n in names]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    for i in range(args.warmup):
        for leg in legs:
            leg.launch(i, sh)
            leg.kernel = g.gemm_last_kernel()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(legs) + 1)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        for li, leg in enumerate(legs):
            leg.launch(s, sh)
            ev[s][li + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    total_ms = ev[0][0].elapsed_time(ev[-1][-1])
    ms_step = total_ms / args.steps
    step_flops = sum(l.flops for l in legs)
    leg_info = {}
    for li, leg in enumerate(legs):
        ms = float(np.mean([ev[s][li].elapsed_time(ev[s][li + 1]) for s in range(args.steps)]))
        peak = rl.mi355x_peak(leg.w.dtype)
        tf = leg.flops / (ms * 1e-3) / 1e12
        leg_info[leg.name] = {"kernel": leg.kernel, "ms": round(ms, 5), "tflops": round(tf, 2),
                              "pct_peak": round(100 * tf * 1e12 / peak, 2),
                              "M": leg.w.M, "N": leg.w.N, "K": leg.w.K, "batch": leg.w.batch,
                              "dtype_in": leg.w.dtype, "gb_per_s": round(leg.bytes / (ms * 1e-3) / 1e9, 1),
                              "input_sets": leg.sets}
        if leg.ws is not None:
            leg_info[leg.name]["workspace_bytes"] = leg.ws_bytes
    roofs = {leg.name: leg_roofline(leg, leg_info[leg.name]) for leg in legs}
    dom = max(legs, key=lambda l: leg_info[l.name]["ms"])
    roof = roofs[dom.name]

    value = step_flops / (ms_step * 1e-3) / 1e12
    dtype = "+".join(sorted({"f32" if l.w.dtype == "f32" else l.w.dtype + "->f32" for l in legs}))
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": args.workload if args.workload != DEFAULT else
                   "4096^3 FP32 GEMM + 4096^3 BF16->FP32 GEMM per step",
                   "legs": leg_info, "algo": args.algo, "epilogue": args.epilogue, "tile_order": args.tile_order,
                   "k_override": args.k,
                   "wall_s": round(wall, 3)},
        "roofline": roof,
        "roofline_legs": roofs,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(legs, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
