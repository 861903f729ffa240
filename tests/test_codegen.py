"""The direct-copy kernels, as compiled for gfx950: their k-loops wait for copies only where the
source says so, and their buffer resources stay in scalar registers.

Each k-loop orders its global->LDS copies with explicit waits (`s_waitcnt vmcnt(N)` in inline
assembly, N the copies allowed in flight) before a plain barrier.  The compiler adds its own
`s_waitcnt vmcnt(0)` before an LDS read when it cannot tell the read from the copies in flight,
which drains every copy, the ones for the next k-tiles included, and serialises the pipeline (an
8-bit build with such waits took 140 us at 4096^3 instead of 59).  This test compiles the kernel
sources to gfx950 assembly on the host (no GPU) and checks every k-loop of every direct-copy
kernel for compiler-generated full waits.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gemm_f32_amd", "csrc")


def _clang():
    for c in ("/opt/rocm/lib/llvm/bin/clang++", shutil.which("amdclang++") or ""):
        if c and os.path.exists(c):
            return c
    pytest.skip("no ROCm clang++ to compile gfx950 assembly")


def _assembly(src: str, tmp_path) -> str:
    out = os.path.join(str(tmp_path), os.path.basename(src) + ".s")
    cmd = [_clang(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "--cuda-device-only", "-S",
           "-x", "hip", os.path.join(CSRC, src), "-o", out]
    if src == "f32_dma.hip":
        cmd[1:1] = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
    subprocess.run(cmd, check=True, capture_output=True)
    return open(out).read()


def _kernels(asm: str, pattern: str):
    """(mangled name, body) of every kernel whose name matches pattern."""
    for m in re.finditer(r"^(_Z\S*" + pattern + r"\S*): ;", asm, re.M):
        start = m.end()
        yield m.group(1), asm[start:asm.index("s_endpgm", start)]


def _loop_bodies(body: str):
    """Instruction lines of each innermost loop: from its header label to the last branch back to it."""
    lines = body.split("\n")
    for i, line in enumerate(lines):
        if "Loop Header" not in line:
            continue
        label = line.split(":")[0].strip()
        back = [j for j in range(i, len(lines)) if "branch" in lines[j] and lines[j].strip().endswith(label)]
        if back:
            yield lines[i:back[-1] + 1]


def _compiler_full_waits(loop) -> int:
    """vmcnt(0) waits outside inline-assembly blocks."""
    n, in_asm = 0, False
    for line in loop:
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
        elif t.startswith(";;#ASMEND"):
            in_asm = False
        elif not in_asm and t.startswith("s_waitcnt") and "vmcnt(0)" in t:
            n += 1
    return n


def _k_loop(loops):
    """The k-loop: the loop with the most matrix instructions."""
    return max(loops, key=lambda lp: sum("v_mfma" in x for x in lp), default=None)


@pytest.mark.parametrize("src,pattern", [("bf16_dma.hip", "k_bf16_dma"), ("f32_dma.hip", "k_f32_dma")])
def test_k_loops_have_no_compiler_full_waits(src, pattern, tmp_path):
    asm = _assembly(src, tmp_path)
    checked = 0
    for name, body in _kernels(asm, pattern):
        loop = _k_loop(list(_loop_bodies(body)))
        if loop is None or not any("v_mfma" in x for x in loop):
            continue                        # the 8-bit build for K < 16 has no k-loop
        assert _compiler_full_waits(loop) == 0, name
        checked += 1
    assert checked >= 8, f"only {checked} k-loops found in {src}"


def _waterfall_loops(body: str) -> int:
    """Loops that step through the lanes' values of a buffer resource: read one lane's resource,
    run the load for the lanes holding the same value, repeat.  The compiler emits them around a
    buffer load whose resource it cannot prove uniform (a strided batch's entry once came out of a
    64-bit division that way), and they serialise every copy."""
    n = 0
    for loop in _loop_bodies(body):
        text = "\n".join(loop)
        if "v_readfirstlane" in text and "s_and_saveexec" in text and "buffer_load" in text:
            n += 1
    return n


@pytest.mark.parametrize("src,pattern", [("bf16_dma.hip", "k_bf16_dma"), ("f32_dma.hip", "k_f32_dma")])
def test_buffer_resources_stay_uniform(src, pattern, tmp_path):
    asm = _assembly(src, tmp_path)
    kernels = list(_kernels(asm, pattern))
    assert len(kernels) >= 8
    for name, body in kernels:
        assert _waterfall_loops(body) == 0, name
