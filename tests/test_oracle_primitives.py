"""Pins of the oracle's numeric primitives (bf16 rounding, exp, sigmoid, SiLU).

Each check compares the oracle against something other than itself: torch's
CPU bf16 cast (a library routine), an exact float64 nearest-value definition,
float64 exp, and closed forms.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O

F32 = np.float32


def _structured_patterns():
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x3FFF, 0x4000, 0x7FFE, 0x7FFF, 0x8000, 0x8001,
                     0xBFFF, 0xC000, 0xFFFE, 0xFFFF], dtype=np.uint32)
    pats = (hi[:, None] | lows[None, :]).reshape(-1)
    rnd = np.random.Generator(np.random.PCG64(1234)).integers(
        0, 1 << 32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([pats, rnd])


def test_bf16_matches_torch_cast_on_all_non_nan_classes():
    u = _structured_patterns()
    f = u.view(F32)
    ok = ~np.isnan(f)
    got = O.bf16_from_f32(f[ok])
    ref = torch.from_numpy(f[ok].copy()).to(torch.bfloat16).view(torch.uint16).numpy()
    assert np.array_equal(got, ref)


def test_bf16_is_nearest_even_by_exact_distance():
    u = _structured_patterns()
    f = u.view(F32)
    f = f[np.isfinite(f)]
    got = O.bf16_from_f32(f)
    uu = f.view(np.uint32)
    lo = (uu >> 16).astype(np.uint32)
    lo_v = (lo << 16).view(F32).astype(np.float64)
    hi = lo + 1
    hi_v = (hi << 16).view(F32).astype(np.float64)  # may be inf at the top
    x = f.astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        d_lo = np.abs(x - lo_v)
        # distance to the next bf16 up; for the largest finite bf16 the "next"
        # is the value 2^128 that IEEE rounding measures against
        top = (lo & 0x7FFF) == 0x7F7F
        hi_mag = np.where(top, 2.0 ** 128, np.abs(hi_v))
        d_hi = np.abs(np.abs(x) - hi_mag)
    choose_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo & 1) == 1))
    ref = np.where(choose_hi, hi, lo).astype(np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("val,bits", [
    (1.0, 0x3F80), (-2.0, 0xC000), (1.0 + 2.0 ** -8, 0x3F80),      # tie -> even
    (1.0 + 3 * 2.0 ** -8, 0x3F82), (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),
    (3.4028234663852886e38, 0x7F80),                                # f32 max -> inf
    (3.3895313892515355e38, 0x7F7F),                                # bf16 max stays
    (0.0, 0x0000), (-0.0, 0x8000), (float("inf"), 0x7F80),
    (2.0 ** -133, 0x0001),                                          # subnormal kept
])
def test_bf16_hand_values(val, bits):
    assert int(O.bf16_from_f32(np.array([val], F32))[0]) == bits


def test_bf16_nan_stays_nan_and_quiet():
    pats = np.array([0x7F800001, 0xFF800001, 0x7FC00000, 0x7FFFFFFF], np.uint32)
    b = O.bf16_from_f32(pats.view(F32))
    back = O.f32_from_bf16(b)
    assert np.all(np.isnan(back))
    assert np.all(b & 0x0040)
    assert np.array_equal(b >> 15, pats >> 31)


def test_bf16_roundtrip_exact():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = O.f32_from_bf16(b)
    keep = ~np.isnan(f)
    assert np.array_equal(O.bf16_from_f32(f[keep]), b[keep])


def _ulp_err(y, x):
    ref = np.exp(x.astype(np.float64))
    ulp = np.spacing(ref.astype(F32)).astype(np.float64)
    return np.abs(y.astype(np.float64) - ref) / ulp


def test_pexp_error_bound_strided_sweep():
    # every 997th f32 pattern whose value lies in the finite-result range
    u = np.arange(0, 1 << 32, 997, dtype=np.uint64).astype(np.uint32)
    x = u.view(F32)
    x = x[np.isfinite(x) & (x >= -87.0) & (x <= 88.0)]
    err = _ulp_err(O.pexp(x), x)
    assert err.max() <= 1.25, err.max()


def test_pexp_error_bound_dense_near_zero_and_routing_range():
    x = np.concatenate([
        np.linspace(-1, 1, 2_000_001, dtype=F32),
        np.linspace(-30, 0, 2_000_001, dtype=F32)])
    err = _ulp_err(O.pexp(x), x)
    assert err.max() <= 1.25, err.max()


def test_pexp_special_cases():
    x = np.array([0.0, -0.0, np.nan, np.inf, -np.inf, 88.0, 88.0001, -87.0, -87.0001], F32)
    y = O.pexp(x)
    assert y[0] == 1.0 and y[1] == 1.0
    assert np.isnan(y[2])
    assert y[3] == np.inf and y[4] == 0.0
    assert np.isfinite(y[5]) and y[6] == np.inf
    assert y[7] >= np.finfo(F32).tiny and y[8] == 0.0
    # results on [-87, 88] are normal numbers
    assert abs(float(y[5]) / math.exp(88.0) - 1) < 1e-6


def test_sigmoid_closed_forms():
    assert O.sigmoid(np.array([0.0], F32))[0] == F32(0.5)
    assert O.sigmoid(np.array([100.0], F32))[0] == F32(1.0)
    assert O.sigmoid(np.array([-100.0], F32))[0] == F32(0.0)
    assert O.sigmoid(np.array([np.inf], F32))[0] == F32(1.0)
    assert O.sigmoid(np.array([-np.inf], F32))[0] == F32(0.0)
    z = np.linspace(-20, 20, 100001, dtype=F32)
    ref = 1.0 / (1.0 + np.exp(-z.astype(np.float64)))
    s = O.sigmoid(z).astype(np.float64)
    assert np.max(np.abs(s - ref) / ref) < 4 * 2.0 ** -24
    # symmetry sigma(z) + sigma(-z) = 1 up to rounding
    assert np.max(np.abs(s + O.sigmoid(-z) - 1.0)) < 2 * 2.0 ** -24


def test_silu_closed_forms():
    g = np.linspace(-20, 20, 100001, dtype=F32)
    ref = g.astype(np.float64) / (1.0 + np.exp(-g.astype(np.float64)))
    s = O.silu(g).astype(np.float64)
    big = np.abs(ref) > 1e-30
    assert np.max(np.abs(s[big] - ref[big]) / np.abs(ref[big])) < 4 * 2.0 ** -24
    assert O.silu(np.array([0.0], F32))[0] == 0.0
    assert O.silu(np.array([100.0], F32))[0] == F32(100.0)
    assert O.silu(np.array([-100.0], F32))[0] == 0.0
