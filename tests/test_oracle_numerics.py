"""Pins for oracle/numerics.py: bf16/fp32 rounding and the comparators.

The rounding is pinned to torch's float32 -> bfloat16 conversion (a library
routine, round to nearest even), to hand-worked ties and boundaries of the
bf16 format, and to a case where direct fp64 -> bf16 rounding must differ from
rounding through fp32.
"""
import numpy as np
import pytest
import torch

from oracle import numerics as N


def torch_bf16(x32):
    return torch.from_numpy(np.asarray(x32, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_round_bf16_matches_torch_on_fp32_values():
    g = np.random.default_rng(123)
    x = np.concatenate([
        g.normal(0, 1, 20000), g.normal(0, 1e-30, 2000), g.normal(0, 1e30, 2000),
        g.uniform(-1e-38, 1e-38, 2000),  # fp32 subnormal / bf16 subnormal range
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-45]),
    ]).astype(np.float32)
    got = N.round_bf16(x.astype(np.float64))
    ref = torch_bf16(x)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_round_bf16_ties_to_even():
    # bf16 spacing at 1 is 2^-7; a half-way value goes to the even neighbour
    assert N.round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert N.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert N.round_bf16(-(1.0 + 2.0 ** -8)) == -1.0
    assert N.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7


def test_round_bf16_is_direct_not_double_rounded():
    # fp32 would round 1 + 2^-8 + 2^-40 onto the tie 1 + 2^-8 (then to 1.0);
    # the exact value is above the tie, so bf16 rounding gives 1 + 2^-7.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert np.float64(np.float32(x)) == 1.0 + 2.0 ** -8
    assert N.round_bf16(x) == 1.0 + 2.0 ** -7


def test_round_bf16_range_ends():
    assert N.round_bf16(N.BF16_MAX) == N.BF16_MAX
    half_ulp_top = 2.0 ** (127 - 8)
    assert np.isinf(N.round_bf16(N.BF16_MAX + half_ulp_top))          # tie -> even -> 2^128 -> inf
    assert N.round_bf16(N.BF16_MAX + half_ulp_top * 0.99) == N.BF16_MAX
    assert N.round_bf16(2.0 ** -133) == 2.0 ** -133                      # smallest subnormal
    assert N.round_bf16(2.0 ** -134) == 0.0                              # tie -> even (0)
    assert N.round_bf16(3 * 2.0 ** -134) == 2.0 ** -132
    assert np.isnan(N.round_bf16(np.nan))
    assert N.round_bf16(-np.inf) == -np.inf


def test_bf16_ulp():
    assert N.bf16_ulp(1.0) == 2.0 ** -7
    assert N.bf16_ulp(1.99) == 2.0 ** -7
    assert N.bf16_ulp(2.0) == 2.0 ** -6
    assert N.bf16_ulp(-0.75) == 2.0 ** -8
    assert N.bf16_ulp(1e-45) == 2.0 ** -133
    assert N.bf16_ulp(0.0) == 2.0 ** -133


def test_ulp_distance_and_floor():
    ref = np.array([[1.0, 0.001, -2.0]])
    got = N.round_bf16(ref)
    assert np.all(N.bf16_ulp_distance(got, ref) == 0)
    # one ulp off at 1.0
    got2 = got.copy()
    got2[0, 0] += 2.0 ** -7
    assert N.bf16_ulp_distance(got2, ref)[0, 0] == 1.0
    # near-zero entry: measured at 2^-8 * row max (= 2^-7 here), whose ulp is 2^-14
    got3 = got.copy()
    got3[0, 1] += 2.0 ** -14
    assert N.bf16_ulp_distance(got3, ref)[0, 1] == pytest.approx(1.0)


def test_round_f32_matches_numpy_cast():
    g = np.random.default_rng(5)
    x = g.normal(0, 1, 1000)
    assert np.array_equal(N.round_f32(x), x.astype(np.float32).astype(np.float64))


def test_comparators():
    ref = np.array([1.0, -4.0, 2.0])
    ok, e = N.check_f32(ref + np.array([0, 4e-5, 0]), ref)
    assert ok and e == pytest.approx(1e-5)
    ok, e = N.check_f32(ref + np.array([0, 4.1e-5, 0]), ref)
    assert not ok
    ok, d = N.check_bf16(N.round_bf16(ref), ref)
    assert ok and d == 0
    ok, e = N.check_matmul(ref * 1.005, ref)
    assert ok
    assert N.frobenius_rel(ref, ref) == 0
