"""Pins of the oracle's MXFP4 quantiser/dequantiser: hand-worked golden blocks,
scale invariants, idempotence, equivariance, error bounds, and the column-wise
definition against a direct column loop."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_blocks.json")


def parse_value(v):
    if isinstance(v, (int, float)):
        return float(v)
    if v == "-0.0":
        return -0.0
    if v == "nan":
        return float("nan")
    if v.startswith("bf16:"):
        return float(F.bf16_bits_to_f64(np.array([int(v[5:], 16)], dtype=np.uint16))[0])
    if "2^" in v:
        mult, _, exp = v.partition("2^")
        m = float(mult.rstrip("*")) if mult else 1.0
        return m * 2.0 ** int(exp)
    raise ValueError(v)


def golden_blocks():
    with open(GOLDEN) as f:
        return json.load(f)["blocks"]


@pytest.mark.parametrize("blk", golden_blocks(), ids=lambda b: b["name"])
def test_golden_blocks(blk):
    x = np.zeros((1, 32))
    vals = [parse_value(v) for v in blk["x"]]
    x[0, :len(vals)] = vals
    packed, scales = mx.mxfp4_quantize_rowwise(x)
    assert int(scales[0, 0]) == blk["scale"]
    codes = mx.unpack_nibbles(packed)[0]
    assert codes[:len(blk["codes"])].tolist() == blk["codes"]
    assert packed[0, :len(blk["packed_prefix"])].tolist() == blk["packed_prefix"]
    assert (codes[len(blk["codes"]):] == 0).all()


def random_blocks(n_blocks, seed):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((n_blocks, 32)).astype(np.float32)
    z *= np.exp2(rng.integers(-60, 60, (n_blocks, 1))).astype(np.float32)
    return torch.from_numpy(z).to(torch.bfloat16).float().double().numpy()


def test_shared_exponent_is_block_max_exponent():
    x = random_blocks(4000, 1)
    _, scales = mx.mxfp4_quantize_rowwise(x)
    for i in range(0, 4000, 7):
        amax = float(np.abs(x[i]).max())
        _, e = math.frexp(amax)  # amax = f * 2^e, f in [0.5, 1)
        assert int(scales[i, 0]) - 127 == max(-127, e - 1 - 2)


def test_scale_invariants_and_bounds():
    x = random_blocks(20000, 2)
    packed, scales = mx.mxfp4_quantize_rowwise(x)
    e = scales.astype(np.int64)[:, 0] - 127
    amax = np.abs(x).max(axis=1)
    ratio = amax * np.exp2(-e.astype(np.float64))
    unclamped = e > -127
    assert ((ratio[unclamped] >= 4) & (ratio[unclamped] < 8)).all()
    v = mx.mxfp4_dequantize_values(packed, scales)
    assert (np.abs(v) <= 6 * np.exp2(e)[:, None]).all()
    # error bound: half a grid step for unsaturated elements, < 2 * 2^E for saturated
    y = np.abs(x) * np.exp2(-e.astype(np.float64))[:, None]
    err = np.abs(v - x) * np.exp2(-e.astype(np.float64))[:, None]
    step = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    sat = y > 6
    assert (err[~sat] <= step[~sat] / 2).all()
    assert (err[sat] < 2).all()


def test_idempotent_and_equivariant():
    x = random_blocks(5000, 3)
    p1, s1 = mx.mxfp4_quantize_rowwise(x)
    v1 = mx.mxfp4_dequantize_values(p1, s1)
    p2, s2 = mx.mxfp4_quantize_rowwise(v1)
    # every unclamped block's largest code is 4 or 6 (amax/2^E lies in [4, 8)), so
    # quantising the dequantised block reproduces scale and codes
    np.testing.assert_array_equal(p1, p2)
    np.testing.assert_array_equal(s1, s2)
    for k in (-5, 3, 17):
        pk, sk = mx.mxfp4_quantize_rowwise(x * 2.0 ** k)
        e1 = s1.astype(np.int64)
        ok = ((e1 + k) > 0) & ((e1 + k) < 255) & (e1 > 0)
        np.testing.assert_array_equal(sk.astype(np.int64)[ok], (e1 + k)[ok])
        okr = ok[:, 0]
        np.testing.assert_array_equal(pk[okr], p1[okr])


def test_nan_inf_blocks():
    x = random_blocks(4, 4)
    x[1, 5] = np.inf
    x[2, 31] = -np.inf
    x[3, 0] = np.nan
    packed, scales = mx.mxfp4_quantize_rowwise(x)
    assert scales[:, 0].tolist()[1:] == [255, 255, 255]
    assert (packed[1:] == 0).all()
    assert scales[0, 0] != 255


def test_colwise_definition_matches_direct_loop():
    rng = np.random.default_rng(6)
    x = random_blocks(64 * 3, 6).reshape(96, 64)[:, :48]  # R=96, C=48
    x[5, 7] = -0.0
    x[40:72, 3] = 0.0
    x[70, 9] = np.nan
    p1, s1 = mx.mxfp4_quantize_colwise(x)
    p2, s2 = mx.mxfp4_quantize_colwise_loops(x)
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(p1, p2)
    assert p1.shape == (48, 48) and s1.shape == (48, 3)


def test_dequantize_exact_in_bf16_and_f32():
    x = random_blocks(3000, 7)
    packed, scales = mx.mxfp4_quantize_rowwise(x)
    v = mx.mxfp4_dequantize_values(packed, scales)
    b = mx.mxfp4_dequantize(packed, scales, "bf16")
    # independent conversion: torch's fp32->bf16 cast of the (exact) values
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(b, ref)
    f = mx.mxfp4_dequantize(packed, scales, "f32")
    np.testing.assert_array_equal(f.view(np.float32).astype(np.float64), v)


def test_dequantize_extreme_scales():
    packed = np.array([[0x87, 0x21] + [0] * 14], dtype=np.uint8)  # codes 7, -0, 1, 2
    for byte, expect in [(0, [6 * 2.0 ** -127, -0.0, 0.5 * 2.0 ** -127, 2.0 ** -127]),
                         (254, [np.inf, -0.0, 2.0 ** 126, 2.0 ** 127]),
                         (255, [np.nan] * 4)]:
        s = np.array([[byte]], dtype=np.uint8)
        f = mx.mxfp4_dequantize(packed, s, "f32").view(np.float32)[0, :4].astype(np.float64)
        np.testing.assert_array_equal(f, np.array(expect))
        b = mx.mxfp4_dequantize(packed, s, "bf16")[0, :4]
        np.testing.assert_array_equal(F.bf16_bits_to_f64(b), np.array(expect))
