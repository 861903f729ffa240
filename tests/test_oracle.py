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
