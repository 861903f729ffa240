"""Each plausible mistake planted in a copy of the oracle must fail at least one pin.

The mutants are built on the CPU from oracle.c with one textual change each; the
unmodified source is never touched.  A mutant that passes every pin would mean the
pins could not tell that mistake from the correct oracle.
"""
import json
import os
import subprocess
import sys
import tempfile

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.library_path()), "oracle.c")

MUTANTS = {
    "drop_last_term": ("for (int64_t k = 0; k < K; ++k) {\n                double a",
                       "for (int64_t k = 0; k < K - 1; ++k) {\n                double a"),
    "skip_first_term": ("for (int64_t k = 0; k < K; ++k) {\n                double a",
                        "for (int64_t k = 1; k < K; ++k) {\n                double a"),
    "transpose_b": ("a * element(B, dtype_b, k, j, ldb, order_b)",
                    "a * element(B, dtype_b, j, k, ldb, order_b)"),
    "wrong_sign": ("s[j] += p;", "s[j] -= p;"),
    "col_major_as_row": ("r * ld + c : r + c * ld", "r * ld + c : r * ld + c"),
    "row_major_as_col": ("r * ld + c : r + c * ld", "r + c * ld : r + c * ld"),
    "bf16_shift": ("<< 16;", "<< 15;"),
    "f16_exponent_bias": ("exp - 25", "exp - 24"),
    "f16_subnormals_as_zero": ("v = ldexp((double)frac, -24);", "v = 0.0;"),
    "f16_fraction_width": ("(double)(1024 + frac)", "(double)(512 + frac)"),
    "scale_without_abs": ("d[j] += fabs(p);", "d[j] += p;"),
    "no_row_reset": ("s[j] = 0.0;\n                d[j] = 0.0;", "d[j] = 0.0;"),
    "fp32_accumulator": ("double p = a * element(B, dtype_b, k, j, ldb, order_b);\n                    s[j] += p;",
                         "double p = a * element(B, dtype_b, k, j, ldb, order_b);\n                    s[j] = (float)(s[j] + p);"),
    "sampled_off_by_one": ("element(B, dtype_b, k, cols[t], ldb, order_b)",
                           "element(B, dtype_b, k, cols[t] > 0 ? cols[t] - 1 : 0, ldb, order_b)"),
    "e4m3_exponent_bias": ("exp - 10);     /* (1 + frac/8)", "exp - 11);     /* (1 + frac/8)"),
    "e4m3_fraction_width": ("ldexp((double)(8 + frac), exp - 10)", "ldexp((double)(4 + frac), exp - 10)"),
    "e4m3_top_exponent_as_nan": ("if (exp == 15 && frac == 7)", "if (exp == 15)"),
    "e4m3_subnormals_as_zero": ("v = ldexp((double)frac, -9);", "v = 0.0;"),
    "e5m2_exponent_bias": ("exp - 17);     /* (1 + frac/4)", "exp - 16);     /* (1 + frac/4)"),
    "e5m2_fraction_width": ("ldexp((double)(4 + frac), exp - 17)", "ldexp((double)(8 + frac), exp - 17)"),
    "e5m2_fields_split_as_e4m3": ("exp = (b >> 2) & 0x1f, frac = b & 0x3;", "exp = (b >> 3) & 0x1f, frac = b & 0x7;"),
    "b_read_with_a_format": ("a * element(B, dtype_b, k, j, ldb, order_b)",
                             "a * element(B, dtype_a, k, j, ldb, order_b)"),
    "mac_undercount": ("count += N;", "count += N - (k == 0);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(before, after)
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        with open(path, "w") as f:
            f.write(mutated)
        lib_path = oracle.build(src=path, out=os.path.join(d, "libmutant.so"))
        # run the pins in a child process: a mutant may read out of bounds and crash
        child = subprocess.run([sys.executable, "-c", _CHILD, lib_path], capture_output=True,
                               text=True, timeout=600, cwd=os.path.dirname(__file__))
        if child.returncode != 0:
            return          # the mistake crashed a pin: detected
        failed = json.loads(child.stdout.strip().splitlines()[-1])
        assert failed, f"mutant {name} passed every pin"


_CHILD = """
import json, os, sys
sys.path.insert(0, os.path.dirname(os.getcwd()))
import oracle, oracle_pins
lib = oracle.oracle.load(sys.argv[1])
failed = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(lib)
    except Exception:
        failed.append(pin.__name__)
print(json.dumps(failed))
"""


# The strided batch and the fused epilogue are written in oracle.py; each plausible mistake in
# either must fail one of their pins.
ORACLE_PY = os.path.join(os.path.dirname(oracle.library_path()), "oracle.py")
PY_MUTANTS = {
    "a_takes_b_stride": ("a = A[z * stride_a:]", "a = A[z * stride_b:]"),
    "b_takes_a_stride": ("b = B[z * stride_b:]", "b = B[z * stride_a:]"),
    "every_entry_reads_entry_0": ("a = A[z * stride_a:]", "a = A[0:]"),
    "entries_shifted": ("C[z], D[z] = gemm(", "C[(z + 1) % batch], D[(z + 1) % batch] = gemm("),
    "gelu_tanh_form": ("Y = pre * 0.5 * (1.0 + erf(pre / np.sqrt(2.0)))",
                       "Y = pre * 0.5 * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (pre + 0.044715 * pre ** 3)))"),
    "bias_per_row": ("b = np.asarray(bias, dtype=np.float64)[None, :]",
                     "b = np.resize(np.asarray(bias, dtype=np.float64), pre.shape[0])[:, None]"),
    "beta_scales_product": ("pre = pre + beta * old", "pre = pre + beta * C"),
    "relu_as_abs": ("Y = np.maximum(pre, 0.0)", "Y = np.abs(pre)"),
    "alpha_dropped": ("pre = alpha * C", "pre = C"),
}


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_batched_mutant_fails_a_pin(name, monkeypatch):
    before, after = PY_MUTANTS[name]
    src = open(ORACLE_PY).read()
    assert src.count(before) == 1, f"mutation site for {name} not found"
    ns = {"__name__": "oracle_mutant", "__file__": ORACLE_PY}
    exec(compile(src.replace(before, after), "oracle_mutant.py", "exec"), ns)
    lib = oracle.oracle.load()
    monkeypatch.setattr(oracle, "gemm_strided_batched", ns["gemm_strided_batched"])
    failed = []
    monkeypatch.setattr(oracle, "epilogue", ns["epilogue"])
    for pin in (oracle_pins.pin_batched_bruteforce, oracle_pins.pin_batched_scaled_identity,
                oracle_pins.pin_epilogue_closed_forms, oracle_pins.pin_gelu_values):
        try:
            pin(lib)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin of oracle.py"
