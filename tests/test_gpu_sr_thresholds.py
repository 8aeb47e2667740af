"""GPU parity of stochastic rounding on inputs placed at the rounding thresholds.

An element rounds up iff its scaled magnitude y exceeds lo + step (r + 1/2) / 2^16,
with r the top 16 bits of its Philox word. Random data almost never lands within a
few ulps of that threshold, so these tensors are built to: every element (fp32)
sits on its own threshold, one ulp below or one ulp above, in every E2M1 interval
including the two below 1. The kernels must still agree with the oracle bit for
bit (their fast decision defers such elements to an exact test). Both random
streams: the per-element words ("sr") and the 16-bit halves ("sr16")."""
import numpy as np
import pytest
import torch

from mxfp4_microscaling_quantization_amd import mxq
from oracle import formats as F
from oracle import mx, nvfp4
from tests.gpu_helpers import assert_equal_bits, f64, require_gpu, sr_stream, u8

pytestmark = pytest.mark.gpu

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def threshold_magnitudes(r16: np.ndarray, rng) -> np.ndarray:
    """y on (or one fp32 ulp around) the SR threshold of a random E2M1 interval."""
    gi = rng.integers(0, 7, r16.shape)
    lo, step = GRID[gi], GRID[gi + 1] - GRID[gi]
    thr = lo + step * (r16.astype(np.float64) + 0.5) / 65536.0
    bits = thr.astype(np.float32).view(np.uint32).astype(np.int64)
    bits += rng.integers(-1, 2, r16.shape)
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("rnd", ["sr", "sr16"])
def test_mxfp4_sr_at_thresholds(rnd):
    dev = require_gpu()
    rng = np.random.default_rng(21)
    R, C, seed, off = 64, 1024, 1234, 8
    r16 = sr_stream(rnd, R, C, seed, off)
    E = rng.integers(-30, 30, (R, C // 32))
    y = threshold_magnitudes(r16, rng)
    y[:, ::32] = 6.0  # block maximum 6 * 2^E fixes the shared exponent at E
    x = np.where(rng.random((R, C)) < 0.5, -1.0, 1.0) * y * np.exp2(np.repeat(E, 32, axis=1))
    xt = torch.from_numpy(x.astype(np.float32))
    assert np.array_equal(f64(xt), x)
    o = mxq.mxq_quantize(xt.to(dev), "mxfp4", "both", rnd, sr_seed=seed, sr_offset=off)
    ref_c, ref_s = mx.mxfp4_quantize_rowwise(x, r16=r16)
    assert np.array_equal(ref_s.astype(np.int64) - 127, E)
    assert_equal_bits(u8(o.scales_row), ref_s, "mx sr thresholds scales")
    assert_equal_bits(u8(o.codes_row), ref_c, "mx sr thresholds codes")
    ref_c, ref_s = mx.mxfp4_quantize_colwise(x, r16_t=sr_stream(rnd, C, R, seed, off))
    assert_equal_bits(u8(o.codes_col), ref_c, "mx sr thresholds col codes")
    assert_equal_bits(u8(o.scales_col), ref_s, "mx sr thresholds col scales")


@pytest.mark.parametrize("rnd", ["sr", "sr16"])
def test_nvfp4_sr_at_thresholds(rnd):
    dev = require_gpu()
    rng = np.random.default_rng(22)
    R, C, seed = 64, 1024, 77
    off = 3 if rnd == "sr" else 16
    r16 = sr_stream(rnd, R, C, seed, off)
    A = 1000.0
    st = float(nvfp4.tensor_scale(A))
    # block scales well inside the E4M3 range; the block maximum sits just above
    # 6 s_b s_t so that it rounds to s_b and no threshold element exceeds it
    codes = rng.integers(16, 118, (R, C // 16))
    sb = F.e4m3_decode(codes)
    y = threshold_magnitudes(r16, rng)
    y = np.minimum(y, 5.5)
    y[:, ::16] = 6.0 * (1 + 2.0 ** -10)
    x = y * np.repeat(sb, 16, axis=1) * st
    x = x.astype(np.float32).astype(np.float64)
    x = np.where(rng.random((R, C)) < 0.5, -1.0, 1.0) * x
    x[0, 1] = A  # the tensor maximum (A / (6 s_t) = 448: block scale 448)
    xt = torch.from_numpy(x.astype(np.float32))
    xg = xt.to(dev)
    amax = mxq.mxq_amax(xg)
    assert float(amax.item()) == nvfp4.tensor_amax(x) == A
    o = mxq.mxq_quantize(xg, "nvfp4", "both", rnd, sr_seed=seed, sr_offset=off, amax=amax)
    ref_c, ref_s, ref_st = nvfp4.nvfp4_quantize_rowwise(x, amax=A, r16=r16)
    # most elements are within a few ulps of their threshold in the exact quotient
    q = np.abs(x) / (np.repeat(F.e4m3_decode(ref_s.astype(np.int64)), 16, axis=1) * float(ref_st))
    gi = np.clip(np.searchsorted(GRID, q, side="right") - 1, 0, 6)
    thr = GRID[gi] + (np.append(GRID, 8.0)[gi + 1] - GRID[gi]) * (r16 + 0.5) / 65536.0
    assert (np.abs(q / thr - 1) < 2.0 ** -20).mean() > 0.5
    assert_equal_bits(u8(o.scales_row), ref_s, "nv sr thresholds block scales")
    assert_equal_bits(u8(o.codes_row), ref_c, "nv sr thresholds codes")
    ref_c, ref_s, _ = nvfp4.nvfp4_quantize_colwise(x, amax=A, r16_t=sr_stream(rnd, C, R, seed, off))
    assert_equal_bits(u8(o.scales_col), ref_s, "nv sr thresholds col block scales")
    assert_equal_bits(u8(o.codes_col), ref_c, "nv sr thresholds col codes")


@pytest.mark.parametrize("rnd", ["sr", "sr16"])
def test_mxfp4_sr_bf16_tiny_values_at_small_random_values(rnd):
    # bf16 blocks: an element's position inside its interval is a whole number of
    # 2^-22 units unless it lies below 2^-16 of the block scale, and then only the
    # random values 0 and 1 put the threshold within reach. Every element whose
    # random value (row-wise, and column-wise through the transposed index) is 0 or
    # 1 gets a tiny bf16 value sitting half a unit above that threshold.
    dev = require_gpu()
    rng = np.random.default_rng(31)
    R, C, seed, off = 512, 2048, 99, 0
    r_row = sr_stream(rnd, R, C, seed, off).astype(np.int64)
    r_col = sr_stream(rnd, C, R, seed, off).astype(np.int64).T  # r of element (r, c) column-wise
    E = rng.integers(-20, 20, (R, C // 32))
    y = rng.uniform(0, 6, (R, C))
    for r_src in (r_row, r_col):
        hit = r_src <= 1
        # 2y 2^22 = 64 r + 32.5: y = (128 r + 65) 2^-24, exact in bf16
        y[hit] = (128 * r_src[hit] + 65) * 2.0 ** -24
    assert (r_row <= 1).sum() + (r_col <= 1).sum() >= 10
    y[:, ::32] = 6.0
    y[:, 16::32] = 6.0  # every 16-row column group of 32 rows holds its maximum too
    y[::32, :] = 6.0
    x = np.where(rng.random((R, C)) < 0.5, -1.0, 1.0) * y * np.exp2(np.repeat(E, 32, axis=1))
    xt = torch.from_numpy(x).to(torch.bfloat16)
    x64 = f64(xt)
    o = mxq.mxq_quantize(xt.to(dev), "mxfp4", "both", rnd, sr_seed=seed, sr_offset=off)
    ref_c, ref_s = mx.mxfp4_quantize_rowwise(x64, r16=sr_stream(rnd, R, C, seed, off))
    assert_equal_bits(u8(o.scales_row), ref_s, f"{rnd} bf16 tiny row scales")
    assert_equal_bits(u8(o.codes_row), ref_c, f"{rnd} bf16 tiny row codes")
    ref_c, ref_s = mx.mxfp4_quantize_colwise(x64, r16_t=sr_stream(rnd, C, R, seed, off))
    assert_equal_bits(u8(o.scales_col), ref_s, f"{rnd} bf16 tiny col scales")
    assert_equal_bits(u8(o.codes_col), ref_c, f"{rnd} bf16 tiny col codes")
