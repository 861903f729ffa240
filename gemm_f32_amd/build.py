"""Build libgemm.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

    python -m gemm_f32_amd.build          # or __graft_entry__.build()

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


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
