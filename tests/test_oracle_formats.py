"""Pins of the oracle's element/scale formats and tensor scale (CPU only).

Each test checks the oracle against something other than itself: the bit
layout of the format, a hand-derived threshold table, torch's float8 and
bfloat16 casts, or ROCm's host-side OCP converters.
"""
import numpy as np
import pytest

from helpers import (E2M1_GRID, dense_f32_patterns, e2m1_by_thresholds, e2m1_signed_values,
                     rocm_encode, rocm_host_converters, torch_bf16_bits, torch_e4m3_encode,
                     torch_e4m3_value)


def test_e2m1_magnitudes_closed_form(orc):
    # E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; largest magnitude 6
    # (the standard NVFP4 target magnitude on the pages).
    vals = np.array([orc.e2m1_value(k) for k in range(16)])
    expect = e2m1_signed_values(np.arange(16, dtype=np.uint8))
    assert np.array_equal(vals, expect)
    assert np.array_equal(vals[:8], E2M1_GRID)
    assert vals[:8].max() == 6.0
    assert np.signbit(vals[8])  # code 0x8 is -0


def test_e2m1_encode_threshold_table(orc):
    y = np.concatenate([dense_f32_patterns(max_exp=255),
                        np.array([np.inf, -np.inf], np.float32)])
    got = orc.e2m1_encode(y)
    exp = e2m1_by_thresholds(y)
    assert np.array_equal(got, exp)


def test_e2m1_encode_rocm_host_library(orc):
    if rocm_host_converters() is None:
        pytest.skip("amdclang++ host-only build of ROCm's OCP converter unavailable")
    y = dense_f32_patterns(max_exp=255)
    rng = np.random.default_rng(7)
    y = np.concatenate([y, rng.standard_normal(1 << 20).astype(np.float32) * 4])
    assert np.array_equal(orc.e2m1_encode(y), rocm_encode("rocm_e2m1", y))


def test_e2m1_grid_is_fixed_point(orc):
    grid = np.concatenate([E2M1_GRID, -E2M1_GRID]).astype(np.float32)
    codes = orc.e2m1_encode(grid)
    assert np.array_equal(e2m1_signed_values(codes), grid)


def test_e4m3_values_match_torch(orc):
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = np.array([orc.e4m3_value(int(c)) for c in codes], np.float32)
    assert np.array_equal(vals, torch_e4m3_value(codes))
    assert orc.e4m3_value(0x7E) == 448.0
    assert orc.e4m3_value(0x01) == 2.0 ** -9
    assert orc.e4m3_value(0x38) == 1.0
    assert np.all(np.diff(vals) > 0)


def test_e4m3_encode_vs_torch_cast(orc):
    t = dense_f32_patterns(signs=(0,), max_exp=255)
    t = t[t <= 448.0]
    rng = np.random.default_rng(3)
    t = np.concatenate([t, (rng.random(1 << 20) * 448).astype(np.float32),
                        np.ldexp(rng.random(1 << 16), -9).astype(np.float32)])
    assert np.array_equal(orc.e4m3_encode(t), torch_e4m3_encode(t))


def test_e4m3_encode_saturates(orc):
    t = np.array([448.0, 448.5, 463.99, 464.0, 480.0, 1e30, np.inf], np.float32)
    assert np.all(orc.e4m3_encode(t) == 0x7E)


def test_e4m3_encode_rocm_host_library(orc):
    if rocm_host_converters() is None:
        pytest.skip("amdclang++ host-only build of ROCm's OCP converter unavailable")
    t = dense_f32_patterns(signs=(0,), max_exp=255)
    t = t[t <= 448.0]
    assert np.array_equal(orc.e4m3_encode(t), rocm_encode("rocm_e4m3", t))


def test_bf16_rne_vs_torch(orc):
    x = dense_f32_patterns(max_exp=255)
    rng = np.random.default_rng(11)
    x = np.concatenate([x, rng.standard_normal(1 << 20).astype(np.float32)])
    assert np.array_equal(orc.bf16_rne(x), torch_bf16_bits(x))


def test_tensor_scales_closed_forms(orc):
    # amax -> 6 * 448 = 2688: the tensor amax lands on the largest E2M1 value
    # times the largest E4M3 value.
    assert orc.tensor_scales(2688.0) == (1.0, 1.0)
    assert orc.tensor_scales(0.0) == (1.0, 1.0)
    e, d = orc.tensor_scales(1.0)
    assert e == np.float32(2688.0)
    assert d == np.float32(np.float64(1.0) / 2688.0)  # correctly rounded quotient
    for k in (-20, -3, 4, 30):
        e2, d2 = orc.tensor_scales(np.ldexp(3.0, k))
        e1, d1 = orc.tensor_scales(3.0)
        assert e2 == np.float32(np.ldexp(np.float64(e1), -k))
        assert d2 == np.float32(np.ldexp(np.float64(d1), k))
