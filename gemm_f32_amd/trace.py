"""Kernel times of libgemm's workloads: rocprofv3 kernel traces of bench.py and their summary.

    python -m gemm_f32_amd.trace collect --out DIR [--only TAG ...]
    python -m gemm_f32_amd.trace table DIR

`collect` runs, for each spec below, one child process

    rocprofv3 --kernel-trace --stats --output-format csv -d DIR/TAG -o r -- \\
        python3 bench.py --no-cpu-baseline --steps S --warmup 3 ARGS

and keeps bench.py's JSON line in DIR/TAG.json.  The spec "default" is the benchmark's own
step, `python3 bench.py --steps 20 --warmup 5` (CPU baseline included).  `table` prints one
markdown row per spec: the kernels rocprofv3 saw (library kernels only) with their dispatch
counts, the kernel time per GEMM call (the sum of the library kernels' durations over the calls
bench.py made: a call that runs a core kernel and an edge strip, or a split-K kernel and its
slab sum, counts all of them), TFLOP/s and compulsory GB/s from that time, and bench.py's own
HIP-event time per call for comparison.

Measurement tooling: it runs rocprofv3 and bench.py as child processes and reads CSV and JSON
files; nothing here is on the GEMM path.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (tag, bench.py arguments, timed steps)
SPECS = [
    ("default", ["--steps", "20", "--warmup", "5"], 20),
    ("square4096_f32", ["--workload", "square4096_f32"], 30),
    ("square4096_f32@MFMA_128x128", ["--workload", "square4096_f32", "--algo", "MFMA_128x128"], 20),
    ("square4096_f32@REGBLOCK", ["--workload", "square4096_f32", "--algo", "REGBLOCK"], 20),
    ("square4096_f32@TILED", ["--workload", "square4096_f32", "--algo", "TILED"], 3),
    ("square4096_f32@NAIVE", ["--workload", "square4096_f32", "--algo", "NAIVE"], 2),
    ("square4096_f32_rc", ["--workload", "square4096_f32_rc"], 20),
    ("square4096_f32_rc@bias_gelu_bf16", ["--workload", "square4096_f32_rc", "--epilogue", "bias_gelu_bf16"], 20),
    ("square4096_bf16", ["--workload", "square4096_bf16"], 30),
    ("square4096_bf16@MFMA_256x128", ["--workload", "square4096_bf16", "--algo", "MFMA_256x128"], 30),
    ("square4096_bf16@MFMA_128x128", ["--workload", "square4096_bf16", "--algo", "MFMA_128x128"], 30),
    ("square4096_f16", ["--workload", "square4096_f16"], 30),
    # both operands row-major (B n-contiguous): the direct-copy kernel's transposing-read build,
    # and the register-staged kernel this layout took before it
    ("square4096_bf16_rr", ["--workload", "square4096_bf16_rr"], 30),
    ("square4096_bf16_rr@MFMA_128x128", ["--workload", "square4096_bf16_rr", "--algo", "MFMA_128x128"], 30),
    ("square4096_bf16_rr@bias_gelu_bf16", ["--workload", "square4096_bf16_rr", "--epilogue", "bias_gelu_bf16"], 30),
    ("square4096_e4m3", ["--workload", "square4096_e4m3"], 30),
    ("square4096_e5m2", ["--workload", "square4096_e5m2"], 30),
    # the same 4096 x 4096 outputs over K: fixed cost (launch, first loads, the 64 MB C write)
    # against the cost per k-tile
    ("square4096_bf16@K128", ["--workload", "square4096_bf16", "--k", "128"], 30),
    ("square4096_bf16@K1024", ["--workload", "square4096_bf16", "--k", "1024"], 30),
    ("square4096_e4m3@K128", ["--workload", "square4096_e4m3", "--k", "128"], 30),
    ("square4096_e4m3@K1024", ["--workload", "square4096_e4m3", "--k", "1024"], 30),
    ("ragged1000_f32", ["--workload", "ragged1000_f32"], 30),
    ("ragged1000_bf16", ["--workload", "ragged1000_bf16"], 30),
    ("ragged4095x4097x1023_f32", ["--workload", "ragged4095x4097x1023_f32"], 30),
    ("ragged4095x4097x1023_bf16", ["--workload", "ragged4095x4097x1023_bf16"], 30),
    ("skinny16x4096x4096_f32", ["--workload", "skinny16x4096x4096_f32"], 30),
    ("skinny16x4096x4096_f32@ws", ["--workload", "skinny16x4096x4096_f32", "--workspace"], 30),
    ("skinny16x4096x4096_bf16", ["--workload", "skinny16x4096x4096_bf16"], 30),
    ("skinny16x4096x4096_bf16@ws", ["--workload", "skinny16x4096x4096_bf16", "--workspace"], 30),
    ("fewcols16x1024x16384_f32@ws", ["--workload", "fewcols16x1024x16384_f32", "--workspace"], 30),
    ("fewcols16x1024x16384_bf16@ws", ["--workload", "fewcols16x1024x16384_bf16", "--workspace"], 30),
    ("fewrows16x8192x4096_f32", ["--workload", "fewrows16x8192x4096_f32"], 30),
    ("shard4096x512x4096_f32", ["--workload", "shard4096x512x4096_f32"], 30),
    ("shard4096x512x4096_f32@ws", ["--workload", "shard4096x512x4096_f32", "--workspace"], 30),
    ("shard4096x512x4096_bf16", ["--workload", "shard4096x512x4096_bf16"], 30),
    ("shard4096x512x4096_bf16@ws", ["--workload", "shard4096x512x4096_bf16", "--workspace"], 30),
    ("llm_attn_proj_2048x4096x4096", ["--workload", "llm_attn_proj_2048x4096x4096"], 30),
    ("llm_attn_proj_2048x4096x4096@identity_f32",
     ["--workload", "llm_attn_proj_2048x4096x4096", "--epilogue", "identity_f32"], 30),
    ("llm_attn_proj_2048x4096x4096@bias_gelu_bf16",
     ["--workload", "llm_attn_proj_2048x4096x4096", "--epilogue", "bias_gelu_bf16"], 30),
    ("llm_ffn_up_2048x11008x4096", ["--workload", "llm_ffn_up_2048x11008x4096"], 30),
    ("llm_ffn_up_2048x11008x4096@identity_f32",
     ["--workload", "llm_ffn_up_2048x11008x4096", "--epilogue", "identity_f32"], 30),
    ("llm_ffn_up_2048x11008x4096@bias_gelu_bf16",
     ["--workload", "llm_ffn_up_2048x11008x4096", "--epilogue", "bias_gelu_bf16"], 30),
    ("llm_ffn_up_2048x11008x4096@beta_bias_relu_f32",
     ["--workload", "llm_ffn_up_2048x11008x4096", "--epilogue", "beta_bias_relu_f32"], 30),
    ("llm_ffn_up_2048x11008x4096_e4m3", ["--workload", "llm_ffn_up_2048x11008x4096_e4m3"], 30),
    ("llm_ffn_down_2048x4096x11008", ["--workload", "llm_ffn_down_2048x4096x11008"], 30),
    ("llm_ffn_down_2048x4096x11008@ws", ["--workload", "llm_ffn_down_2048x4096x11008", "--workspace"], 30),
    ("attn_scores_32x2048x2048x128_bf16", ["--workload", "attn_scores_32x2048x2048x128_bf16"], 30),
    ("attn_pv_32x2048x128x2048_bf16", ["--workload", "attn_pv_32x2048x128x2048_bf16"], 30),
    # the tile scheduler's remaps off (entries' tiles spread over the XCDs in dispatch order)
    ("attn_pv_32x2048x128x2048_bf16@rowmajor",
     ["--workload", "attn_pv_32x2048x128x2048_bf16", "--tile-order", "rowmajor"], 30),
]


def collect(args) -> None:
    os.makedirs(args.out, exist_ok=True)
    for tag, bench_args, steps in SPECS:
        if args.only and tag not in args.only:
            continue
        if tag == "default":
            bench = bench_args
        else:
            bench = ["--no-cpu-baseline", "--steps", str(steps), "--warmup", "3", *bench_args]
        d = os.path.join(args.out, tag)
        cmd = ["timeout", "-k", "10", "300", "rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv",
               "-d", d, "-o", "r", "--", sys.executable, os.path.join(ROOT, "bench.py"), *bench]
        print("+", " ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
        if r.returncode != 0 or not lines:
            sys.stderr.write(r.stdout[-2000:] + r.stderr[-2000:])
            raise SystemExit(f"{tag}: status {r.returncode}")
        with open(os.path.join(args.out, tag + ".json"), "w") as f:
            f.write(lines[-1] + "\n")


def _stats(d: str) -> list:
    f = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not f:
        return []
    return [r for r in csv.DictReader(open(f[0], newline="")) if "gemm::" in r["Name"]]


def _short(name: str) -> str:
    s = name.replace("void ", "").replace("gemm::(anonymous namespace)::", "")
    return s.split("(std::conditional")[0].split("(gemm::")[0].split("(float*")[0]


def table(args) -> None:
    sys.path.insert(0, ROOT)
    import gemm_inputs as gi
    from gemm_f32_amd import roofline as rl
    print("| spec | bench arguments | library kernel (bench.py) | rocprofv3 kernels: dispatches x average µs | "
          "kernel µs per call | TFLOP/s | % of peak (dtype) | compulsory GB/s | bench.py events µs per call |")
    print("|---|---|---|---|---|---|---|---|---|")
    for tag, bench_args, steps in SPECS:
        d = os.path.join(args.dir, tag)
        jf = d + ".json"
        if not os.path.exists(jf):
            continue
        out = json.load(open(jf))
        rows = _stats(d)
        legs = out["config"]["legs"]
        calls = out["steps"] + out["warmup"]
        arg = " ".join(bench_args)
        if tag == "default":
            # one row per leg: the FP32 leg's kernels are k_f32_*, the 16-bit leg's k_bf16_*
            for name, leg in legs.items():
                w = gi.WORKLOADS[name]
                fam = "k_f32" if w.dtype == "f32" else "k_bf16"
                mine = [r for r in rows if _short(r["Name"]).startswith(fam)]
                us = sum(int(r["Calls"]) * float(r["AverageNs"]) for r in mine) / 1e3 / calls
                _row(f"default: {name}", arg, leg, mine, us, w, rl)
            continue
        (name, leg), = legs.items()
        w = gi.WORKLOADS[name]
        us = sum(int(r["Calls"]) * float(r["AverageNs"]) for r in rows) / 1e3 / calls
        _row(tag, arg, leg, rows, us, w, rl)


def _row(tag, arg, leg, rows, us, w, rl) -> None:
    kern = "; ".join(f"`{_short(r['Name'])}` {r['Calls']} x {float(r['AverageNs']) / 1e3:.1f}" for r in rows)
    M, N, K, batch = leg["M"], leg["N"], leg["K"], leg["batch"]      # as run (K may be overridden)
    tf = 2 * batch * M * N * K / (us * 1e-6) / 1e12
    e = 4 if w.dtype == "f32" else 1 if w.dtype in ("e4m3", "e5m2", "e4m3_e5m2", "e5m2_e4m3") else 2
    gbs = batch * (e * (M * K + K * N) + 4 * M * N) / (us * 1e-6) / 1e9
    pct = 100 * tf * 1e12 / rl.mi355x_peak(w.dtype)
    print(f"| {tag} | `{arg}` | {leg['kernel']} | {kern} | {us:.1f} | {tf:.1f} | {pct:.1f} | {gbs:.0f} | "
          f"{leg['ms'] * 1e3:.1f} |")


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("collect")
    c.add_argument("--out", required=True)
    c.add_argument("--only", nargs="*", default=None)
    t = sub.add_parser("table")
    t.add_argument("dir")
    args = ap.parse_args()
    {"collect": collect, "table": table}[args.cmd](args)


if __name__ == "__main__":
    main()
