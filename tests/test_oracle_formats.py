"""Pins of the oracle's number-format codecs against things other than itself:
torch's E4M3 and bf16 casts, hand-derived closed-form rounding tables, and exact
rational brute force."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F


def all_bf16_finite_nonneg():
    bits = np.arange(0, 0x7F80, dtype=np.uint16)  # +0 .. largest finite
    return bits, F.bf16_bits_to_f64(bits)


def test_e2m1_grid_from_bit_fields():
    # the E2M1 grid the format definition yields (and that the method statement lists)
    assert F.E2M1_MAGNITUDES.tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert F.e2m1_value(0b1111) == -6.0 and F.e2m1_value(0b1001) == -0.5
    assert np.signbit(F.e2m1_decode(np.array([8])))[0]  # code 0x8 is -0


def test_e2m1_grid_exact_in_e4m3():
    g = torch.tensor(np.concatenate([F.E2M1_MAGNITUDES, -F.E2M1_MAGNITUDES]), dtype=torch.float32)
    back = g.to(torch.float8_e4m3fn).to(torch.float32)
    assert torch.equal(back, g)


def closed_form_e2m1(y):
    """Hand-derived decision table for nearest-even E2M1 with saturation."""
    y = np.asarray(y)
    code = np.zeros(y.shape, dtype=np.int64)
    code += (y > 0.25)
    code += (y >= 0.75)
    code += (y > 1.25)
    code += (y >= 1.75)
    code += (y > 2.5)
    code += (y >= 3.5)
    code += (y > 5.0)
    return code


@pytest.mark.parametrize("shift", [-130, -8, -3, -2, -1, 0, 1, 2, 3, 10, 125])
def test_e2m1_rounding_all_bf16_closed_form(shift):
    _, v = all_bf16_finite_nonneg()
    y = np.ldexp(v, shift)  # exact in float64
    got = F.e2m1_round_nearest_even(y).astype(np.int64)
    np.testing.assert_array_equal(got, closed_form_e2m1(y))


def _fraction_nearest_even(y: Fraction) -> int:
    grid = [Fraction(v) for v in F.E2M1_MAGNITUDES.tolist()]
    d = [abs(y - g) for g in grid]
    m = min(d)
    cands = [i for i, di in enumerate(d) if di == m]
    if len(cands) == 1:
        return cands[0]
    return [c for c in cands if c % 2 == 0][0]


def test_e2m1_rounding_fraction_bruteforce():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 0x7F80, 4000).astype(np.uint16)
    v = F.bf16_bits_to_f64(bits)
    for shift in (-1, 0, 2, 5):
        y = np.ldexp(v, shift)
        got = F.e2m1_round_nearest_even(y)
        for yi, gi in zip(y.tolist(), got.tolist()):
            assert gi == _fraction_nearest_even(Fraction(yi)), yi


def test_e2m1_ties_and_saturation():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    # ties go to the even code: 0.25->0, 0.75->1.0, 1.25->1.0, 1.75->2.0, 2.5->2.0, 3.5->4.0, 5->4.0
    assert F.e2m1_round_nearest_even(mids).tolist() == [0, 2, 2, 4, 4, 6, 6]
    assert F.e2m1_round_nearest_even(np.array([6.0, 7.0, 1e30, 5.0000001])).tolist() == [7, 7, 7, 7]


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F.e4m3_decode(np.arange(256))
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))
    assert F.E4M3_MAX == 448.0


def test_e4m3_encode_matches_torch_below_464():
    # torch's fp32 -> float8_e4m3fn cast is round-to-nearest-even; it only differs
    # from the saturating encoder at |v| >= 464 (torch gives NaN there).
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_bits_to_f64(bits)
    keep = np.isfinite(v) & (np.abs(v) < 464)
    rng = np.random.default_rng(3)
    extra = (rng.standard_normal(200000) * np.exp(rng.uniform(-12, 6, 200000))).astype(np.float32)
    v = np.concatenate([v[keep], extra.astype(np.float64)[np.abs(extra) < 464]])
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = F.e4m3_round_nearest_even(v)
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_saturation_and_nan():
    out = F.e4m3_round_nearest_even(np.array([464.0, 1e9, -np.inf, np.nan, -0.0]))
    assert out.tolist() == [0x7E, 0x7E, 0xFE, 0x7F, 0x80]


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    mant = rng.integers(0, 1 << 23, 300000)
    exp = rng.integers(0, 255, 300000)
    sign = rng.integers(0, 2, 300000)
    b32 = ((sign << 31) | (exp << 23) | mant).astype(np.uint32)
    v32 = b32.view(np.float32)
    ref = torch.from_numpy(v32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = F.round_f64_to_bf16_bits(v32.astype(np.float64))
    np.testing.assert_array_equal(ours, ref)


def test_bf16_rounding_is_single_rounding():
    # a float64 value just above a bf16 midpoint that fp32 would round onto the
    # midpoint: single rounding must go up
    mid = 1.0 + 2.0 ** -8  # midpoint between 1 and 1 + 2^-7
    v = np.array([mid + 2.0 ** -40, mid, mid - 2.0 ** -40, 1.0 + 3 * 2.0 ** -8])
    got = F.round_f64_to_bf16_bits(v)
    assert got.tolist() == [0x3F81, 0x3F80, 0x3F80, 0x3F82]
    assert F.round_f64_to_bf16_bits(np.array([2.0 ** 128, -3e38 * 1.2, np.nan])).tolist() == [0x7F80, 0xFF80, 0x7FC0]
