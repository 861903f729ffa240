"""The clock probe (gemm_f32_amd.clockprobe) instruments copies of the two direct-copy kernel
sources by inserting timestamps at fixed places.  These host tests check that every place is still
found in the current sources, exactly where intended, and that nothing else in the text changes."""
import os

from gemm_f32_amd import clockprobe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gemm_f32_amd", "csrc")


def _check(src, fn, tag):
    text = open(os.path.join(CSRC, src)).read()
    out = fn(text)
    # three timestamps, one record, one read-back function; the original text is a subsequence
    assert out.count("__builtin_amdgcn_s_memtime()") == 3
    assert out.count(f"g_clk_{tag}[idx]") == 1
    assert f'extern "C" int gemm_probe_read_{tag}' in out
    it = iter(out.splitlines())
    assert all(any(ln == o for o in it) for ln in text.splitlines()), "an original line was changed"
    # the entry stamp is inside the kernel that owns the record, before its k-loop end stamp
    i0, i1, i2 = out.index("P0_t ="), out.index("P1_t ="), out.index("P2_t =")
    assert i0 < i1 < i2


def test_bf16_anchors():
    _check("bf16_dma.hip", clockprobe.instrument_bf16, "bf16")


def test_f32_anchors():
    _check("f32_dma.hip", clockprobe.instrument_f32, "f32")
