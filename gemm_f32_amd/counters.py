"""Hardware-counter evidence for libgemm's kernels: rocprofv3 passes over bench.py and their summary.

    python -m gemm_f32_amd.counters collect --workload W --out DIR [--tile-order rowmajor] [--algo A]
    python -m gemm_f32_amd.counters calibrate --out DIR
    python -m gemm_f32_amd.counters summarize --calib DIR DIR... [--traffic-json profiles/traffic.json]

`collect` runs three rocprofv3 passes, each a child process `rocprofv3 --pmc ... -- python3 bench.py
--workload W --steps 3 --warmup 1 --no-cpu-baseline` (one counter set per pass, within the per-pass
limits of the counter blocks):
  A  MfmaUtil, VALUBusy, LDSBankConflict (rocprofv3's derived percentages) and the raw SQ_INSTS_MFMA,
     SQ_INSTS_VALU, SQ_INSTS_LDS, SQ_WAVES, SQ_BUSY_CU_CYCLES;
  B  FETCH_SIZE (KiB the L2s fetched from the fabric: last-level cache or HBM) and TCC_HIT_sum;
  C  WRITE_SIZE (KiB written) with TCC_MISS_sum and TCC_REQ_sum;
  D  cycle counts (GRBM_GUI_ACTIVE, SQ_BUSY_CU_CYCLES, the matrix-core busy cycles, the waves' resident
     and waiting cycles) in a run that also traces each dispatch's start and end (--kernel-trace): the
     CUs' busy cycles, the share of them the matrix cores worked, and a lower bound on the shader clock
     (the clock itself: gemm_f32_amd/clockprobe.py).
`calibrate` runs passes B and C over bench.py's plain 256 MiB device copy, whose bytes are known:
FETCH_SIZE and WRITE_SIZE of a kernel are scaled by (bytes copied) / (what the copy's counters read).
`summarize` averages every library kernel's counters over its dispatches and prints one markdown row
per kernel: matrix-core and vector-ALU busy, LDS bank-conflict stalls, L2 hit rate, HBM bytes per
launch (scaled) against the compulsory bytes of the workload; and, where pass D was collected, a second
table of clock and cycles per kernel.  `--workload default` profiles bench.py's default step (the FP32
and the BF16 4096^3 GEMM, interleaved).

This is measurement tooling: it runs rocprofv3 and bench.py as child processes and reads CSV files;
nothing here is on the GEMM path.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import subprocess
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PASSES = {
    "A": ["MfmaUtil", "VALUBusy", "LDSBankConflict", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS",
          "SQ_WAVES", "SQ_BUSY_CU_CYCLES"],
    "B": ["FETCH_SIZE", "TCC_HIT_sum"],
    "C": ["WRITE_SIZE", "TCC_MISS_sum", "TCC_REQ_sum"],
    "D": ["GRBM_GUI_ACTIVE", "GRBM_COUNT", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_WAVE_CYCLES",
          "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_LDS"],
}
# passes that also record each dispatch's start and end
TRACED = {"D"}
COPY_BYTES = 256 * 1024 * 1024        # bench.py --copy-calibration: one 256 MiB device copy


def _run_pass(tag: str, counters: list, bench_args: list, out: str) -> None:
    d = os.path.join(out, tag)
    trace = ["--kernel-trace"] if tag.rsplit("_", 1)[-1] in TRACED else []
    cmd = ["timeout", "-s", "KILL", "120", "rocprofv3", *trace, "--pmc", *counters, "--output-format", "csv",
           "-d", d, "-o", "run", "--", sys.executable, os.path.join(ROOT, "bench.py"), *bench_args]
    print("+", " ".join(cmd), flush=True)
    r = subprocess.run(cmd)
    if r.returncode != 0:
        raise SystemExit(f"pass {tag} failed with status {r.returncode}")


def collect(args) -> None:
    bench = (["--workload", args.workload] if args.workload != "default" else []) + [
        "--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--tile-order", args.tile_order]
    if args.algo:
        bench += ["--algo", args.algo]
    stem = f"{args.workload}@{args.tile_order}" + (f"~{args.algo}" if args.algo else "")
    for tag in args.passes:
        _run_pass(f"{stem}_{tag}", PASSES[tag], bench, args.out)


def calibrate(args) -> None:
    for tag in ("B", "C"):
        _run_pass(f"copy_{tag}", PASSES[tag], ["--copy-calibration", "--steps", "3", "--warmup", "1"], args.out)


def _read(dir_: str) -> dict:
    """{kernel name: {counter: [value per dispatch]}} from the counter CSV files under dir_."""
    vals: dict = defaultdict(lambda: defaultdict(dict))
    for f in glob.glob(os.path.join(dir_, "**", "*counter_collection.csv"), recursive=True):
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                vals[row["Kernel_Name"]][row["Counter_Name"]][row["Dispatch_Id"]] = float(row["Counter_Value"])
    return {k: {c: list(d.values()) for c, d in v.items()} for k, v in vals.items()}


def _read_dispatches(dir_: str) -> dict:
    """{kernel name: [(counters of one dispatch, duration ns, waves)]} from a traced counter run."""
    durs = {}
    for f in glob.glob(os.path.join(dir_, "**", "*kernel_trace.csv"), recursive=True):
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                durs[row["Dispatch_Id"]] = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
    disp: dict = defaultdict(dict)
    for f in glob.glob(os.path.join(dir_, "**", "*counter_collection.csv"), recursive=True):
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                d = disp[(row["Kernel_Name"], row["Dispatch_Id"])]
                d[row["Counter_Name"]] = float(row["Counter_Value"])
                d["_waves"] = int(row["Grid_Size"]) // 64
    out: dict = defaultdict(list)
    for (k, did), c in disp.items():
        if did in durs:
            out[k].append((c, durs[did], c.pop("_waves")))
    return out


def _agent(dir_: str) -> dict:
    for f in glob.glob(os.path.join(dir_, "**", "*agent_info.csv"), recursive=True):
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                if row.get("Name", "").startswith("gfx"):
                    return {"xcc": int(row["Num_Xcc"]), "simds": int(row["Simd_Count"]),
                            "mhz": float(row["Max_Engine_Clk_Fcompute"])}
    return {"xcc": 8, "simds": 1024, "mhz": 2400.0}


def clock_table(dirs: list) -> None:
    """Pass D: per kernel, the cycles its CUs were busy and how much of them the matrix cores worked.

    SQ_BUSY_CU_CYCLES (summed over the CUs) counts only cycles in which a CU holds a wavefront of the
    kernel, so busy cycles per CU over the kernel's traced duration are a lower bound on the shader
    clock.  GRBM_GUI_ACTIVE (summed over the XCDs) also counts the profiler's counter window around the
    dispatch, about 21 k cycles per dispatch on this machine: a short kernel shows it as more cycles
    than its duration allows, so it is reported but not turned into a clock."""
    print("\n| workload | tile order | kernel | dispatches | kernel µs | GRBM cycles per XCD (incl. counter window) | "
          "CU-busy cycles per CU | clock lower bound GHz (busy cycles / kernel time) | "
          "matrix busy % of CU-busy cycles | wave cycles waiting % |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for d in dirs:
        stem = os.path.basename(os.path.normpath(d))[:-2]
        workload, order = stem.split("@")
        ag = _agent(d)
        cus = ag["simds"] // 4
        for k, rows in sorted(_read_dispatches(d).items()):
            if not _library_kernel(k):
                continue
            grbm = _mean([c["GRBM_GUI_ACTIVE"] / ag["xcc"] for c, _, _ in rows])
            dur = _mean([t for _, t, _ in rows])
            busy = _mean([c["SQ_BUSY_CU_CYCLES"] / cus for c, _, _ in rows])
            low = _mean([c["SQ_BUSY_CU_CYCLES"] / cus / t for c, t, _ in rows])
            mfma = _mean([c["SQ_VALU_MFMA_BUSY_CYCLES"] / ag["simds"] / (c["SQ_BUSY_CU_CYCLES"] / cus) for c, _, _ in rows])
            wait = _mean([c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"] for c, _, _ in rows])
            print(f"| {workload} | {order.replace('~', ', algo ')} | `{_short(k)}` | {len(rows)} | {dur / 1e3:.1f} | {grbm:.0f} | {busy:.0f} | {low:.3f} | "
                  f"{100 * mfma:.1f} | {100 * wait:.1f} |")


def _mean(x):
    return sum(x) / len(x) if x else float("nan")


def _library_kernel(name: str) -> bool:
    return "gemm::" in name


def _short(name: str) -> str:
    """Kernel template name without its long argument list."""
    s = name.replace("void ", "").replace("gemm::(anonymous namespace)::", "")
    return s.split("(std::conditional")[0].split("(gemm::")[0]


def summarize(args) -> None:
    calib = {}
    for tag, ctr in (("B", "FETCH_SIZE"), ("C", "WRITE_SIZE")):
        data = _read(os.path.join(args.calib, f"copy_{tag}"))
        v = [_mean(d[ctr]) for k, d in data.items() if ctr in d and "copyBuffer" in k]
        if not v:
            raise SystemExit(f"no copy kernel with {ctr} under {args.calib}")
        calib[ctr] = COPY_BYTES / 1024 / v[0]
    print(f"Calibration (256 MiB device copy): FETCH_SIZE x {calib['FETCH_SIZE']:.4f}, "
          f"WRITE_SIZE x {calib['WRITE_SIZE']:.4f}\n")
    sys.path.insert(0, ROOT)
    import gemm_inputs as gi
    print("| workload | tile order | kernel | MFMA busy % | VALU busy % | LDS bank-conflict % | L2 hit % | "
          "FETCH KiB | WRITE KiB | HBM bytes/launch (scaled) | compulsory bytes | ratio |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    traffic = {}
    for base in args.dirs:
        tagged = os.path.basename(os.path.normpath(base))
        if not tagged.endswith("_A"):
            continue
        stem = tagged[:-2]
        workload, order = stem.split("@")          # order[~algo]: an explicitly chosen algorithm
        w = gi.WORKLOADS.get(workload)
        if w is None:                              # the default step: two workloads, clock table only
            continue
        e = 4 if w.dtype == "f32" else 1 if w.dtype in gi.FP8_DTYPES else 2
        compulsory = w.batch * (e * (w.M * w.K + w.K * w.N) + 4 * w.M * w.N)
        parts = {t: _read(os.path.join(os.path.dirname(os.path.normpath(base)), f"{stem}_{t}")) for t in "ABC"}
        names = sorted({k for p in parts.values() for k in p if _library_kernel(k)})
        for k in names:
            a, b, c = (parts[t].get(k, {}) for t in "ABC")
            fetch, write = _mean(b.get("FETCH_SIZE", [])), _mean(c.get("WRITE_SIZE", []))
            hit, miss = _mean(b.get("TCC_HIT_sum", [])), _mean(c.get("TCC_MISS_sum", []))
            hbm = fetch * 1024 * calib["FETCH_SIZE"] + write * 1024 * calib["WRITE_SIZE"]
            print(f"| {workload} | {order.replace('~', ', algo ')} | `{_short(k)}` | {_mean(a.get('MfmaUtil', [])):.1f} | "
                  f"{_mean(a.get('VALUBusy', [])):.1f} | {_mean(a.get('LDSBankConflict', [])):.2f} | "
                  f"{100 * hit / (hit + miss):.1f} | {fetch:.0f} | {write:.0f} | {hbm:.4e} | {compulsory:.4e} | "
                  f"{hbm / compulsory:.3f} |")
            traffic[(workload, order, k)] = (fetch, write, hbm, compulsory)
    if args.traffic_json:
        _update_traffic(args.traffic_json, traffic, calib)
    clocks = [os.path.join(os.path.dirname(os.path.normpath(b)), os.path.basename(os.path.normpath(b))[:-2] + "_D")
              for b in args.dirs if os.path.basename(os.path.normpath(b))[-2:] in ("_A", "_D")]
    clocks = [d for d in clocks if os.path.isdir(d)]
    if clocks:
        clock_table(clocks)


def _update_traffic(path: str, traffic: dict, calib: dict) -> None:
    """Record HBM bytes per launch of the dominant kernel of each workload measured in the default
    tile order, keyed by the library's name for the kernel the default choice runs (gemm_plan) and
    the workload, with the digest of the kernel's sources (bench.py reports the figure only while
    the digest still matches)."""
    sys.path.insert(0, ROOT)
    import bench
    import gemm_f32_amd as g
    import gemm_inputs as gi
    rec = json.load(open(path)) if os.path.exists(path) else {}
    by_workload: dict = defaultdict(list)
    for (workload, order, k), v in traffic.items():
        if order == "swizzled":
            by_workload[workload].append(v)
    for workload, items in by_workload.items():
        w = gi.WORKLOADS[workload]
        if w.batch > 1:
            continue
        fetch, write, hbm, compulsory = max(items)          # the kernel that moves the most
        lib = g.gemm_plan(w.dtype, w.M, w.N, w.K, w.order_a, w.order_b, w.order_c)[0]
        rec[f"{lib}@{workload}"] = {
            "hbm_bytes_per_launch": int(hbm), "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
            "fetch_scale": round(calib["FETCH_SIZE"], 4), "write_scale": round(calib["WRITE_SIZE"], 4),
            "compulsory_bytes": compulsory, "ratio_to_compulsory": round(hbm / compulsory, 3),
            "source_digest": bench.kernel_source_digest(lib)}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("collect")
    c.add_argument("--workload", required=True)
    c.add_argument("--algo", default=None)
    c.add_argument("--tile-order", default="swizzled", choices=["swizzled", "rowmajor"])
    c.add_argument("--out", required=True)
    c.add_argument("--passes", default="ABCD", help="counter passes to run (letters of A, B, C, D)")
    k = sub.add_parser("calibrate")
    k.add_argument("--out", required=True)
    s = sub.add_parser("summarize")
    s.add_argument("--calib", required=True)
    s.add_argument("--traffic-json", default=None)
    s.add_argument("dirs", nargs="+", help="the pass-A (or pass-D) directories (…/<workload>@<order>_A)")
    args = ap.parse_args()
    {"collect": collect, "calibrate": calibrate, "summarize": summarize}[args.cmd](args)


if __name__ == "__main__":
    main()
