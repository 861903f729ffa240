"""CPU pins of the fp64 oracle and of the seeded input generator (no GPU)."""
import math

import numpy as np
import pytest

import gemm_inputs as gi
import oracle
import oracle_pins


@pytest.fixture(scope="module")
def lib():
    return oracle.oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin, lib):
    pin(lib)


def test_normalised_error_metric():
    ref = np.array([[1.0, -2.0], [0.0, 4.0]])
    D = np.array([[2.0, 4.0], [0.0, 8.0]])
    assert oracle.normalised_error(ref, ref, D) == 0.0
    t = ref + np.array([[1e-6, 0.0], [0.0, -8e-6]])
    assert math.isclose(oracle.normalised_error(t, ref, D), 1e-6, rel_tol=1e-9)
    # where D == 0 the value must be exactly zero; -0 counts as zero
    t = ref.copy(); t[1, 0] = -0.0
    assert oracle.normalised_error(t, ref, D) == 0.0
    t[1, 0] = 1e-30
    assert oracle.normalised_error(t, ref, D) == math.inf
    t = ref.copy(); t[0, 0] = np.nan
    assert oracle.normalised_error(t, ref, D) == math.inf
    t = ref.copy(); t[0, 1] = np.inf
    assert oracle.normalised_error(t, ref, D) == math.inf


def test_bf16_rounding_is_nearest_even():
    # hand-worked bit patterns: 1 + 2^-8 is a tie between 0x3F80 and 0x3F81 -> even 0x3F80;
    # 1 + 3*2^-8 ties between 0x3F81 and 0x3F82 -> even 0x3F82; 1 + 2^-8 + 2^-20 rounds up.
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20, -2.5,
                  3.4e38, -0.0], dtype=np.float32)
    bits = gi.f32_to_bf16_bits(x)
    assert [int(b) for b in bits] == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x7F80, 0x8000]
    assert np.isnan(gi.bf16_bits_to_f32(gi.f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]
    # widening is exact and round-tripping a bf16 value is the identity
    r = np.random.default_rng(0).integers(0, 0x7F80, 1000).astype(np.uint16)
    assert np.array_equal(gi.f32_to_bf16_bits(gi.bf16_bits_to_f32(r)), r)


def test_fp8_rounding_is_nearest_even():
    """fp32 -> OCP E4M3 / E5M2 rounding of the input generator: hand-worked ties and edges, and
    agreement with torch's float8 conversions (a library routine) on 200 000 random values."""
    import torch
    # E4M3: 1 + 2^-4 ties between 1.0 (0x38) and 1.125 (0x39) -> even 0x38; 1 + 3*2^-4 ties
    # between 0x39 and 0x3A -> even 0x3A; 464 ties between 448 (0x7E) and the NaN code -> 0x7E;
    # 500 overflows to NaN; 2^-10 ties between 0 and the smallest subnormal 2^-9 -> 0
    x = np.array([1.0, 1.0625, 1.1875, 464.0, 500.0, 2.0 ** -10, 3 * 2.0 ** -11, -0.0, -448.0], np.float32)
    assert [int(b) for b in gi.f32_to_fp8_bits(x, "e4m3")] == [0x38, 0x38, 0x3A, 0x7E, 0x7F, 0x00, 0x01, 0x80, 0xFE]
    # E5M2: 61440 ties between 57344 (0x7B) and 65536 (overflow) -> infinity 0x7C; 2^-17 -> 0
    x = np.array([1.0, 1.125, 61440.0, -70000.0, 2.0 ** -17, 2.0 ** -16, np.inf], np.float32)
    assert [int(b) for b in gi.f32_to_fp8_bits(x, "e5m2")] == [0x3C, 0x3C, 0x7C, 0xFC, 0x00, 0x01, 0x7C]
    r = np.random.default_rng(1).standard_normal(200000).astype(np.float32) * np.float32(50.0)
    for fmt, tdt in (("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)):
        ours = gi.f32_to_fp8_bits(r, fmt)
        theirs = torch.from_numpy(r).to(tdt).view(torch.uint8).numpy()
        dec = gi.fp8_bits_to_f32(ours, fmt)
        assert np.array_equal(ours[~np.isnan(dec)], theirs[~np.isnan(dec)])
        assert np.all(np.isnan(torch.from_numpy(theirs[np.isnan(dec)]).view(tdt).float().numpy()))
        # widening is exact: round-tripping every finite pattern is the identity
        allb = np.arange(256, dtype=np.uint16).astype(np.uint8)
        fin = np.isfinite(gi.fp8_bits_to_f32(allb, fmt))
        back = gi.f32_to_fp8_bits(gi.fp8_bits_to_f32(allb[fin], fmt), fmt)
        assert np.array_equal(back, allb[fin])


def test_layout_places_elements():
    L = np.arange(12, dtype=np.float32).reshape(3, 4)
    flat, ld = gi.lay_out(L, gi.ROW_MAJOR, 6)
    assert ld == 6 and flat[1 * 6 + 2] == L[1, 2] and np.isnan(flat[4])
    flat, ld = gi.lay_out(L, gi.COL_MAJOR, 5)
    assert ld == 5 and flat[1 + 2 * 5] == L[1, 2] and np.isnan(flat[3])
    assert np.array_equal(gi.unpack_c(gi.lay_out(L, gi.COL_MAJOR, 5)[0], 3, 4, 5, gi.COL_MAJOR), L)


def test_seeds_are_reproducible_and_distinct():
    a = gi.make_problem(8, 9, 10, "f32", wid=3)
    b = gi.make_problem(8, 9, 10, "f32", wid=3)
    c = gi.make_problem(8, 9, 10, "f32", wid=4)
    assert np.array_equal(a.A, b.A) and np.array_equal(a.B, b.B)
    assert not np.array_equal(a.A_logical, c.A_logical)
    assert not np.array_equal(a.A_logical[:8, :9], a.B_logical[:8, :9])
    llm = gi.make_problem(64, 64, 256, "f32", dist="llm", wid=5)
    assert 0.8 < llm.A_logical.std() < 1.2 and 0.015 < llm.B_logical.std() < 0.025
    u = gi.make_problem(64, 64, 64, "f32", wid=6)
    assert u.A_logical.min() >= -1 and u.A_logical.max() <= 1
