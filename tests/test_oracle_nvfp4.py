"""Pins of the oracle's NVFP4 quantiser: exact rational (Fraction) brute force of
every rounding it takes, the tensor-scale landing on 448, error bounds, special
cases, and statistical checks of stochastic rounding."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import mx, nvfp4, philox


def fr_round_to_fp32(q: Fraction) -> float:
    """Exact round-to-nearest-even of a positive rational to fp32 (normal or subnormal)."""
    if q == 0:
        return 0.0
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 23)
    n = round(q / quantum)  # Python rounds Fractions half to even
    return float(n * quantum)


def fr_nearest_even(q: Fraction, grid) -> int:
    g = [Fraction(v) for v in grid]
    if q >= g[-1]:
        return len(g) - 1
    d = [abs(q - v) for v in g]
    m = min(d)
    c = [i for i, di in enumerate(d) if di == m]
    return c[0] if len(c) == 1 else [i for i in c if i % 2 == 0][0]


def test_tensor_scale_is_correctly_rounded():
    rng = np.random.default_rng(0)
    amaxes = np.concatenate([
        F.bf16_bits_to_f64(rng.integers(1, 0x7F80, 3000).astype(np.uint16)),
        rng.standard_normal(3000).astype(np.float32).astype(np.float64) * 2.0 ** rng.integers(-140, 120, 3000),
    ])
    amaxes = np.abs(amaxes[np.isfinite(amaxes) & (amaxes != 0)])
    for a in amaxes:
        ref = fr_round_to_fp32(Fraction(float(a)) / 2688)
        assert float(nvfp4.tensor_scale(float(a))) == ref, a


def test_quotient_roundings_match_exact_rationals():
    # random and adversarial (near-midpoint) element / scale combinations
    rng = np.random.default_rng(1)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    cases = []
    for _ in range(3000):
        x = float(F.bf16_bits_to_f64(np.array([rng.integers(0x3000, 0x5000)], dtype=np.uint16))[0])
        sb = float(F.E4M3_MAGNITUDES[rng.integers(1, 127)])
        st = float(np.float32(rng.uniform(0.5, 1) * 2.0 ** rng.integers(-30, 10)))
        cases.append((x, sb, st))
        # an s_t that puts x right at (or next to) a midpoint
        m = mids[rng.integers(0, 7)]
        st_mid = np.float32(x / (m * sb))
        for k in (-2, -1, 0, 1, 2):
            cases.append((x, sb, float(np.nextafter(st_mid, np.float32(np.inf) if k > 0 else np.float32(0))
                                       if k else st_mid) if abs(k) == 1 else float(st_mid)))
    for x, sb, st in cases:
        y = abs(x) / (sb * st)
        got = int(F.e2m1_round_nearest_even(np.array([y]))[0])
        ref = fr_nearest_even(Fraction(x) / (Fraction(sb) * Fraction(st)), F.E2M1_MAGNITUDES.tolist())
        assert got == ref, (x, sb, st)
        # the E4M3 block-scale quotient
        q = abs(x) / (6.0 * st)
        got8 = int(F.e4m3_round_nearest_even(np.array([q]))[0])
        ref8 = fr_nearest_even(Fraction(x) / (6 * Fraction(st)), F.E4M3_MAGNITUDES.tolist())
        assert got8 == ref8, (x, st)


def bf16_matrix(rows, cols, seed):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((rows, cols)).astype(np.float32)
    z *= np.exp(rng.uniform(-4, 4, (rows, 1))).astype(np.float32)
    return torch.from_numpy(z).to(torch.bfloat16).double().numpy()


def test_amax_block_lands_on_448_and_6():
    x = bf16_matrix(64, 256, 2)
    p, sb, st = nvfp4.nvfp4_quantize_rowwise(x)
    r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert sb[r, c // 16] == 0x7E  # 448
    assert mx.unpack_nibbles(p)[r, c] & 7 == 7  # 6.0
    assert (sb & 0x7F).max() == 0x7E


def test_codes_and_scales_against_exact_rationals_small():
    x = bf16_matrix(4, 64, 3)
    p, sb, st = nvfp4.nvfp4_quantize_rowwise(x)
    A = Fraction(float(np.abs(x).max()))
    assert float(st) == fr_round_to_fp32(A / 2688)
    codes = mx.unpack_nibbles(p)
    for r in range(4):
        for b in range(4):
            blk = x[r, b * 16:(b + 1) * 16]
            ab = Fraction(float(np.abs(blk).max()))
            k = fr_nearest_even(ab / (6 * Fraction(float(st))), F.E4M3_MAGNITUDES.tolist())
            assert sb[r, b] == k
            den = Fraction(float(F.E4M3_MAGNITUDES[k])) * Fraction(float(st))
            for i in range(16):
                v = blk[i]
                m = fr_nearest_even(Fraction(abs(float(v))) / den, F.E2M1_MAGNITUDES.tolist())
                assert codes[r, b * 16 + i] == (m | (8 if np.signbit(v) else 0))


def test_reconstruction_error_bound():
    x = bf16_matrix(128, 512, 4)
    p, sb, st = nvfp4.nvfp4_quantize_rowwise(x)
    v = nvfp4.nvfp4_dequantize_values(p, sb, st)
    den = (F.e4m3_decode(sb) * np.float64(st))[..., None]
    y = (np.abs(x).reshape(128, 32, 16) / den)
    err = np.abs(v - x).reshape(128, 32, 16) / den
    step = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    ok = y <= 6
    assert (err[ok] <= step[ok] / 2).all()


def test_special_tensors():
    z = np.zeros((2, 32))
    z[1, 3] = -0.0
    p, sb, st = nvfp4.nvfp4_quantize_rowwise(z)
    assert st == 0 and (sb == 0).all() and mx.unpack_nibbles(p)[1, 3] == 8
    x = bf16_matrix(2, 32, 5)
    x[0, 0] = np.nan
    p, sb, st = nvfp4.nvfp4_quantize_rowwise(x)
    assert np.isnan(st) and (sb == 0x7F).all() and (p == 0).all()
    # a tiny block next to a huge one: its scale underflows E4M3 -> sign bits only
    x = np.zeros((1, 32))
    x[0, 0] = 2.0 ** 20
    x[0, 16:] = -(2.0 ** -10)
    p, sb, st = nvfp4.nvfp4_quantize_rowwise(x)
    assert sb[0, 1] == 0 and (mx.unpack_nibbles(p)[0, 16:] == 8).all()


def test_dequantize_single_rounding():
    x = bf16_matrix(16, 64, 6)
    p, sb, st = nvfp4.nvfp4_quantize_rowwise(x)
    v = nvfp4.nvfp4_dequantize_values(p, sb, st)
    f = nvfp4.nvfp4_dequantize(p, sb, st, "f32").view(np.float32)
    np.testing.assert_array_equal(f, v.astype(np.float32))
    b = nvfp4.nvfp4_dequantize(p, sb, st, "bf16")
    for i in range(0, v.size, 37):
        ref = fr_round_to_fp32(Fraction(abs(float(v.flat[i]))))
        # bf16: 8 significant bits; check against an exact rational rounding
        q = Fraction(abs(float(v.flat[i])))
        if q == 0:
            continue
        e = q.numerator.bit_length() - q.denominator.bit_length()
        while Fraction(2) ** e > q:
            e -= 1
        while Fraction(2) ** (e + 1) <= q:
            e += 1
        quantum = Fraction(2) ** (max(e, -126) - 7)
        exact = float(round(q / quantum) * quantum)
        got = abs(float(F.bf16_bits_to_f64(b.flat[i:i + 1])[0]))
        assert got == exact
        assert ref >= 0


@pytest.mark.parametrize("stream", ["words", "halves"])
@pytest.mark.parametrize("which", ["nvfp4", "mxfp4"])
def test_stochastic_rounding_statistics(which, stream):
    rng = np.random.default_rng(7)
    # one block repeated: fixed scales, many random draws
    row = np.concatenate([[6.0], rng.uniform(-6, 6, 15)])
    row = torch.from_numpy(row).to(torch.bfloat16).double().numpy()
    reps = 4096
    x = np.tile(row, (reps, 2))  # [reps, 32]
    r16 = (philox.tensor_r16 if stream == "words" else philox.tensor_r16_halves)(reps, 32, seed=7)
    if which == "nvfp4":
        p, sb, st = nvfp4.nvfp4_quantize_rowwise(x, r16=r16)
        v = nvfp4.nvfp4_dequantize_values(p, sb, st)
        den = float(F.e4m3_decode(sb[0:1, 0])[0]) * float(st)
        assert (sb == sb[0, 0]).all()
    else:
        p, s = mx.mxfp4_quantize_rowwise(x, r16=r16)
        v = mx.mxfp4_dequantize_values(p, s)
        den = 2.0 ** (int(s[0, 0]) - 127)
        assert (s == s[0, 0]).all()
    y = np.abs(row) / den
    g = F.E2M1_MAGNITUDES
    lo = np.clip(np.searchsorted(g, y, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    frac = np.where(hi > lo, (y - g[lo]) / np.maximum(g[hi] - g[lo], 1e-300), 0.0)
    mags = np.abs(v[:, :16]) / den
    up = (mags > g[lo] + 1e-12).mean(axis=0)
    on = (mags == g[lo]) | (mags == g[hi])
    assert on.all()  # always one of the two neighbours
    sd = np.sqrt(frac * (1 - frac) / reps) + 1e-12
    assert (np.abs(up - frac) <= 5 * sd + 2.0 ** -16).all()
    # unbiased: mean of dequantised values equals the input within 5 sigma
    mean = v[:, :16].mean(axis=0)
    step = (g[hi] - g[lo]) * den
    assert (np.abs(mean - row) <= 5 * step * sd + step * 2.0 ** -16).all()


def test_stochastic_rounding_keeps_grid_values():
    x = np.tile(np.array([0.0, 0.5, -1.0, 1.5, 2.0, -3.0, 4.0, 6.0] * 2), (64, 1))
    r16 = philox.tensor_r16(64, 16, seed=1)
    p, sb, st = nvfp4.nvfp4_quantize_rowwise(x, r16=r16)
    p0, sb0, st0 = nvfp4.nvfp4_quantize_rowwise(x)
    np.testing.assert_array_equal(p, p0)


def test_2d_equals_1d_when_every_row_block_holds_the_tile_maximum():
    # when each 1x16 row block of a 16x16 tile reaches the tile's maximum, the 2D
    # block amax equals every 1D block amax, so both quantisations coincide
    rng = np.random.default_rng(4)
    R, C = 48, 64
    x = rng.standard_normal((R, C))
    tmax = np.exp2(rng.integers(-3, 4, (R // 16, C // 16))) * 3.0
    x = np.clip(x, -2.9, 2.9) * np.repeat(np.repeat(tmax / 3.0, 16, 0), 16, 1)
    pos = rng.integers(0, 16, (R, C // 16))
    for r in range(R):
        for b in range(C // 16):
            x[r, 16 * b + pos[r, b]] = tmax[r // 16, b] * (1 if (r + b) % 2 else -1)
    c2, s2, st2 = nvfp4.nvfp4_quantize_2d(x)
    c1, s1, st1 = nvfp4.nvfp4_quantize_rowwise(x)
    assert st1 == st2
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_2d_transpose_symmetry_and_tile_constant_scales():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((64, 96)) * np.exp(rng.uniform(-3, 3, (64, 1)))
    c, s, st = nvfp4.nvfp4_quantize_2d(x)
    ct, stt, stt_t = nvfp4.nvfp4_quantize_2d(x.T)
    assert st == stt_t
    assert np.array_equal(mx.unpack_nibbles(ct), mx.unpack_nibbles(c).T)
    # the scales are constant within a tile, and the transpose's are the transpose
    tiles = s.reshape(4, 16, 6)
    assert (tiles == tiles[:, :1, :]).all()
    assert np.array_equal(stt[::16], s[::16].T)


def test_2d_single_tile_by_hand():
    # one 16x16 tile holding the tensor maximum A = 10.5, so s_t = A / 2688 = 2^-8 is
    # exact and s_b = 448 (byte 0x7E); an element then codes as E2M1(6 |x| / A)
    x = np.zeros((16, 16))
    x[0, 0] = 10.5       # 6                      -> code 7
    x[5, 7] = -5.25      # 3                      -> code 5, negative
    x[9, 3] = 2.625      # 1.5                    -> code 3
    x[15, 15] = 1.3125   # 0.75, a tie of 0.5 and 1 -> even: 1.0, code 2
    x[2, 2] = 0.4375     # 0.25, a tie of 0 and 0.5 -> even: 0, code 0
    c, s, st = nvfp4.nvfp4_quantize_2d(x)
    assert st == np.float32(2.0 ** -8) and (s == 0x7E).all()
    g = mx.unpack_nibbles(c)
    assert g[0, 0] == 7 and g[5, 7] == 0x8 | 5 and g[9, 3] == 3 and g[15, 15] == 2 and g[2, 2] == 0
    assert (np.delete(g.reshape(-1), [0, 5 * 16 + 7, 9 * 16 + 3, 255]) == 0).all()
