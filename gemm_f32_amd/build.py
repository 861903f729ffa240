"""Build libgemm.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

    python -m gemm_f32_amd.build          # or __graft_entry__.build()
    python -m gemm_f32_amd.build --resource-table    # markdown table of the last build's report

Each source compiles to an object under gemm_f32_amd/_build/ (in parallel), then they
link into gemm_f32_amd/libgemm.so.  The compiler's per-kernel resource report (VGPRs,
AGPRs, LDS bytes, scratch/spills, occupancy) is written to _build/resource_usage.txt.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgemm.so")

SOURCES = ["api.hip", "fill.hip", "f32_ladder.hip", "f32_regblock.hip", "f32_mfma.hip", "f32_dma.hip",
           "bf16_mfma.hip", "bf16_dma.hip", "skinny.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed FP32 vector instructions stay off (the compiler would otherwise form them
    # from plain float code); the FP32 roof is reached through the matrix cores instead
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-source extra flags.  The FP32 direct-copy kernel keeps its matrix accumulators in
# ordinary vector registers: with the accumulation-register form the compiler rotated the
# accumulators through register copies on every k-tile (visible in the kernel's assembly).
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
EXTRA_FLAGS = {"f32_dma.hip": _VGPR_FORM}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: libgemm needs ROCm's hipcc to build")


def _compile(src: str) -> tuple[str, str]:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [hipcc(), *FLAGS, *EXTRA_FLAGS.get(src, []), "-Rpass-analysis=kernel-resource-usage", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj, r.stderr


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libgemm.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    report = "\n".join(_resource_lines(log) for _, log in results)
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        f.write(report)
    tmp = LIB + ".tmp"
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(report)
    return LIB


def _resource_lines(log: str) -> str:
    keep = []
    for line in log.splitlines():
        m = re.search(r"remark: (.*)", line)
        if m and "[-Rpass-analysis=kernel-resource-usage]" in line:
            keep.append(m.group(1).replace(" [-Rpass-analysis=kernel-resource-usage]", ""))
    return "\n".join(keep)


def _first_template_arg(name: str) -> str:
    """`k<Cfg<1, 2>, true, 3>(...)` -> `k<Cfg<1, 2>, ...>`: a kernel and its tile configuration."""
    if "<" not in name:
        return name.split("(")[0]
    i = name.index("<") + 1
    depth = 1
    for j in range(i, len(name)):
        c = name[j]
        depth += c == "<"
        depth -= c == ">"
        if depth == 0 or (depth == 1 and c == ","):
            return name[:j] + (", ...>" if c == "," else ">")
    return name


def resource_table(path: str = os.path.join(BUILD, "resource_usage.txt")) -> str:
    """Markdown table of the compiler's resource report for the last build, one row per kernel
    template and tile configuration (ranges over its instantiations): registers, LDS, scratch and
    spills, occupancy."""
    text = open(path).read()
    blocks = re.split(r"^Function Name: ", text, flags=re.M)[1:]
    rows = []
    for b in blocks:
        lines = b.splitlines()
        fields = dict(re.match(r"\s*(.*?):\s*(.*)", ln).groups() for ln in lines[1:] if ":" in ln)
        rows.append((lines[0].strip(), fields))
    names = subprocess.run(["c++filt"], input="\n".join(n for n, _ in rows), capture_output=True,
                           text=True).stdout.splitlines() if shutil.which("c++filt") else [n for n, _ in rows]
    groups: dict = {}
    for (_, f), name in zip(rows, names):
        short = name.replace("void ", "").replace("gemm::(anonymous namespace)::", "").replace("gemm::", "")
        groups.setdefault(_first_template_arg(short), []).append(f)

    def rng(fs, key):
        v = sorted({int(f.get(key, 0)) for f in fs})
        return str(v[0]) if len(v) == 1 else f"{v[0]}-{v[-1]}"

    out = ["| kernel (tile configuration) | instantiations | VGPRs | AGPRs | SGPRs | LDS bytes | scratch bytes/lane | "
           "VGPR spills | SGPR spills | occupancy (waves/SIMD) |", "|---|---|---|---|---|---|---|---|---|---|"]
    for k, fs in groups.items():
        out.append(f"| `{k}` | {len(fs)} | {rng(fs, 'VGPRs')} | {rng(fs, 'AGPRs')} | {rng(fs, 'TotalSGPRs')} | "
                   f"{rng(fs, 'LDS Size [bytes/block]')} | {rng(fs, 'ScratchSize [bytes/lane]')} | "
                   f"{rng(fs, 'VGPRs Spill')} | {rng(fs, 'SGPRs Spill')} | {rng(fs, 'Occupancy [waves/SIMD]')} |")
    return "\n".join(out)


if __name__ == "__main__":
    if "--resource-table" in sys.argv:
        print(resource_table())
    else:
        print(build(verbose="-v" in sys.argv))
