"""GPU parity of every variant of the Hadamard-transform + MXFP4 kernels on inputs
whose butterfly sums are exact in fp32 (small integers times powers of two, with a
per-row power so that column chunks mix binades): bf16 and fp32 input, nearest-even
and stochastic rounding, row-wise, column-wise and both. The transform is then exact
on both sides, so codes and scales must match the oracle bit for bit, apart from
the sign of an exact zero (the oracle's float64 sums and the fp32 butterfly may
reach zero with either sign)."""
import numpy as np
import pytest
import torch

from gpu_helpers import f64, require_gpu, sr_stream, u8
from mxfp4_microscaling_quantization_amd import mxq
from oracle import mx, rht

pytestmark = pytest.mark.gpu

R, C = 96, 416
SEED, OFFSET, OFFSET16 = 21, 6, 8


def check(codes, scales, y, r16, what):
    ref_c, ref_s = mx.mxfp4_quantize_rowwise(y, r16=r16)
    assert np.array_equal(scales, ref_s), what + " scales"
    g, r = mx.unpack_nibbles(codes), mx.unpack_nibbles(ref_c)
    assert np.array_equal(g & 7, r & 7), what + " code magnitudes"
    nz = y != 0
    assert np.array_equal((g >> 3)[nz], (r >> 3)[nz]), what + " code signs"


@pytest.mark.parametrize("axis", ["row", "col", "both"])
@pytest.mark.parametrize("rnd", ["rne", "sr", "sr16"])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_rht_mxfp4_variants_exact_inputs(dt, rnd, axis):
    dev = require_gpu()
    rng = np.random.default_rng(17)
    x = rng.integers(-64, 65, (R, C)) * np.exp2(rng.integers(-3, 4, (R, 1)) - 4.0)
    xt = torch.from_numpy(x).to(dt)
    assert np.array_equal(f64(xt), x)  # exact in both input types
    mask = rht.sign_mask_from_seed(13)
    off = OFFSET16 if rnd == "sr16" else OFFSET
    o = mxq.mxq_rht_quantize_mask(xt.to(dev), mask, "mxfp4", axis, rnd, sr_seed=SEED, sr_offset=off)
    what = f"{dt} {rnd} {axis}"
    if axis in ("row", "both"):
        r16 = sr_stream(rnd, R, C, SEED, off)
        check(u8(o.codes_row), u8(o.scales_row), rht.rht_rowwise(x, mask), r16, what + " row")
    if axis in ("col", "both"):
        r16t = sr_stream(rnd, C, R, SEED, off)
        check(u8(o.codes_col), u8(o.scales_col), rht.rht_rowwise(x.T.copy(), mask), r16t, what + " col")


@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("rnd", ["rne", "sr", "sr16"])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_rht_nvfp4_variants_exact_inputs(dt, rnd, axis):
    # the tensor scale belongs to the transformed tensor: its amax (exact here) goes
    # to both sides, and every NVFP4 decision is then taken on exact values
    dev = require_gpu()
    rng = np.random.default_rng(19)
    x = rng.integers(-64, 65, (R, C)) * np.exp2(rng.integers(-3, 4, (R, 1)) - 4.0)
    xt = torch.from_numpy(x).to(dt)
    xg = xt.to(dev)
    mask = rht.sign_mask_from_seed(14)
    amax = mxq.mxq_rht_amax(xg, mask, axis)
    a_ref = rht.rht_amax(x, mask, axis)
    assert float(amax.item()) == a_ref
    off = OFFSET16 if rnd == "sr16" else OFFSET
    o = mxq.mxq_rht_quantize_mask(xg, mask, "nvfp4", axis, rnd, sr_seed=SEED, sr_offset=off, amax=amax)
    if axis == "row":
        r16 = sr_stream(rnd, R, C, SEED, off)
        ref_c, ref_s, st = rht.rht_nvfp4_rowwise(x, mask, a_ref, r16)
        y, codes, scales = rht.rht_rowwise(x, mask), u8(o.codes_row), u8(o.scales_row)
    else:
        r16t = sr_stream(rnd, C, R, SEED, off)
        ref_c, ref_s, st = rht.rht_nvfp4_colwise(x, mask, a_ref, r16t)
        y, codes, scales = rht.rht_rowwise(x.T.copy(), mask), u8(o.codes_col), u8(o.scales_col)
    what = f"nvfp4 {dt} {rnd} {axis}"
    assert float(o.tensor_scale.item()) == float(st), what + " tensor scale"
    assert np.array_equal(scales, ref_s), what + " scales"
    g, r = mx.unpack_nibbles(codes), mx.unpack_nibbles(ref_c)
    assert np.array_equal(g & 7, r & 7), what + " code magnitudes"
    nz = y != 0
    assert np.array_equal((g >> 3)[nz], (r >> 3)[nz]), what + " code signs"
