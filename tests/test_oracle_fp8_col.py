"""Pins of the oracle's MXFP4-rows -> FP8-columns conversion (reading F4): torch's
E4M3 cast on whole 128-token groups, a Fraction brute force over ragged expert
segments (empty, tiny and partial groups, NaN and zero blocks, extreme scale
bytes), the closed form of each group's largest element, and losslessness when a
group's exponents are close."""
from fractions import Fraction

import numpy as np
import torch

from oracle import fp8, mx

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def random_mx(rng, R, C, e_lo=110, e_hi=140, p_zero=0.15):
    codes = rng.integers(0, 16, (R, C)).astype(np.uint8)
    codes[rng.random((R, C)) < p_zero] &= 0x8
    e = rng.integers(e_lo, e_hi, (R, C // 32)).astype(np.uint8)
    return mx.pack_nibbles(codes), e, codes


def e4m3_fraction(k: int) -> Fraction:
    """Value of a 7-bit E4M3 magnitude code from its bit fields (bias 7, 3 mantissa bits)."""
    e, m = k >> 3, k & 7
    if e == 0:
        return Fraction(m, 8) * Fraction(1, 2 ** 6)
    return (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


GRID = [e4m3_fraction(k) for k in range(127)]  # 0x7F is NaN


def nearest_even_e4m3(y: Fraction) -> int:
    best = min(range(127), key=lambda k: (abs(GRID[k] - y), k & 1))
    return best


def brute_force(codes, e, offsets):
    """Scalar Fraction reference written from the definition, group by group."""
    R, C = codes.shape
    val = {}
    for r in range(R):
        for c in range(C):
            b = int(e[r, c // 32])
            if b == 255:
                val[r, c] = None
                continue
            m = int(codes[r, c])
            v = Fraction(E2M1[m & 7]).limit_denominator() * Fraction(2) ** (b - 127)
            val[r, c] = (-v if m & 8 else v, bool(m & 8))
    q8 = np.zeros((C, R), np.uint8)
    scales = []
    for ei in range(len(offsets) - 1):
        for t0 in range(offsets[ei], offsets[ei + 1], 128):
            t1 = min(t0 + 128, offsets[ei + 1])
            col_scales = []
            for c in range(C):
                items = [val[t, c] for t in range(t0, t1)]
                if any(it is None for it in items):
                    q8[c, t0:t1] = 0x7F
                    col_scales.append(0x7FC00000)
                    continue
                amax = max(abs(v) for v, _ in items)
                k = 0
                if amax > 0:
                    k = -200
                    while amax > 448 * Fraction(2) ** k:
                        k += 1
                for i, (v, neg) in enumerate(items):
                    code = nearest_even_e4m3(abs(v) / Fraction(2) ** k)
                    q8[c, t0 + i] = code | (0x80 if neg else 0)
                col_scales.append(int(np.array([2.0 ** k], np.float32).view(np.uint32)[0]))
            scales.append(col_scales)
    return q8, np.array(scales, np.uint32).T.reshape(C, -1)


def test_expert_group_offsets():
    # counts 0, 1, 129, 256, 0, 128 -> groups 0, 1, 2, 2, 0, 1
    np.testing.assert_array_equal(fp8.expert_group_offsets([0, 0, 1, 130, 386, 386, 514]),
                                  [0, 0, 1, 3, 5, 5, 6])


def test_single_expert_whole_groups_match_torch_cast():
    rng = np.random.default_rng(0)
    R, C = 256, 64
    packed, e, codes = random_mx(rng, R, C)
    q8, s = fp8.mxfp4_rows_to_fp8_cols(packed, e, [0, R])
    # torch: values from the E2M1 table and the scale bytes, transpose, 128-groups,
    # k from frexp, E4M3 by torch's round-to-nearest-even cast
    mag = torch.tensor(E2M1, dtype=torch.float64)[torch.from_numpy(codes & 7).long()]
    sign = torch.where(torch.from_numpy(codes & 8) > 0, -1.0, 1.0).double()
    sc = torch.pow(2.0, torch.from_numpy(e.astype(np.int64) - 127).double()).repeat_interleave(32, dim=1)
    xt = (mag * sign * sc).T.reshape(C, R // 128, 128)
    amax = xt.abs().amax(-1)
    m, ex = torch.frexp(amax)  # amax = m 2^ex, m in [0.5, 1)
    k = (ex - 1 - 8).double()
    k = torch.where(amax / torch.pow(2.0, k) > 448, k + 1, k)
    ref = (xt / torch.pow(2.0, k)[..., None]).to(torch.float8_e4m3fn).view(torch.uint8).reshape(C, R)
    np.testing.assert_array_equal(q8, ref.numpy())
    np.testing.assert_array_equal(s, torch.pow(2.0, k).float().numpy().view(np.uint32))


def test_ragged_experts_brute_force():
    rng = np.random.default_rng(1)
    counts = [0, 1, 5, 0, 130, 128, 3]
    offsets = np.concatenate([[0], np.cumsum(counts)]).tolist()
    R, C = offsets[-1], 32
    packed, e, codes = random_mx(rng, R, C)
    e[7, 0] = 255        # a NaN block inside expert 4's first group
    codes[150:170] &= 8  # signed zeros
    e[200, 0] = 0        # smallest scale byte (values down to 2^-128)
    e[201, 0] = 254      # largest finite scale byte
    e[2, 0] = 1
    packed = mx.pack_nibbles(codes)
    q8, s = fp8.mxfp4_rows_to_fp8_cols(packed, e, offsets)
    rq, rs = brute_force(codes, e, offsets)
    np.testing.assert_array_equal(q8, rq)
    np.testing.assert_array_equal(s, rs)


def test_group_maximum_closed_form_and_scale():
    # the largest element of a group is (1 + f/2) 2^F and lands on 256 or 384 (codes
    # 0x78 / 0x7C) under s = 2^(F - 8)
    rng = np.random.default_rng(2)
    R, C = 384, 32
    packed, e, codes = random_mx(rng, R, C)
    q8, s = fp8.mxfp4_rows_to_fp8_cols(packed, e, [0, 100, 384])
    x = mx.mxfp4_dequantize_values(packed, e).T
    gofs = 0
    for t0, t1 in ((0, 100), (100, 228), (228, 356), (356, 384)):
        seg = np.abs(x[:, t0:t1])
        amax = seg.max(axis=1)
        F = np.floor(np.log2(amax)).astype(np.int64)
        np.testing.assert_array_equal(s[:, gofs], np.ldexp(1.0, F - 8).astype(np.float32).view(np.uint32))
        top = q8[np.arange(C), t0 + seg.argmax(axis=1)] & 0x7F
        assert set(np.unique(top)) <= {0x78, 0x7C}
        gofs += 1


def test_lossless_when_group_exponents_are_close():
    # every nonzero element within 2^-16 of its group's top binade is exactly
    # representable after the shift (normal down to 2^-6, subnormal steps 2^-9)
    rng = np.random.default_rng(3)
    R, C = 256, 64
    packed, e, codes = random_mx(rng, R, C, e_lo=120, e_hi=127)
    q8, s = fp8.mxfp4_rows_to_fp8_cols(packed, e, [0, 128, 256])
    x = mx.mxfp4_dequantize_values(packed, e).T
    sv = s.view(np.float32).astype(np.float64)
    back = fp8.e4m3_decode(q8) * np.repeat(sv, 128, axis=1)
    np.testing.assert_array_equal(back, x)


def test_lossy_subnormal_tail_rounds_to_nearest_even():
    # column 0 holds a group maximum of 2^0 (F = 0, s = 2^-8) and two elements
    # 2^-17 below it: 1.0 and 1.5 quanta of 2^-9 after the shift -> 1 and 2 (tie to even)
    codes = np.zeros((3, 32), np.uint8)
    e = np.full((3, 1), 127, np.uint8)
    codes[:, 0] = [2, 2, 3]   # 1.0, 1.0, 1.5
    e[1:, 0] = 127 - 17
    q8, s = fp8.mxfp4_rows_to_fp8_cols(mx.pack_nibbles(codes), e, [0, 3])
    assert s[0, 0] == np.float32(2.0 ** -8).view(np.uint32)
    assert list(q8[0]) == [0x78, 0x01, 0x02]
