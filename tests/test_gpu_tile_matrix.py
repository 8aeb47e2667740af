"""GPU parity of every variant of the column-wise (and fused row + column) tile kernel
without a transform: bf16 and fp32 input, MXFP4 and NVFP4, nearest-even and
stochastic rounding, column-wise only and both outputs, on a shape whose tiles are
ragged in both directions, bit-exact against the oracle. Column-wise stochastic
rounding indexes the transpose: element (r, c) draws word n = offset + c * R + r."""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_equal_bits, bits32, f64, require_gpu, sr_stream, u8
from mxfp4_microscaling_quantization_amd import mxq
from oracle import mx, nvfp4

pytestmark = pytest.mark.gpu

R, C = 288, 416  # 2 full 128-row tiles + 32 rows; 1 full 256- or 3 full 128-column tiles + the rest
SEED, OFFSET, OFFSET16 = 5, 12345, 12344  # word stream: an offset that is not a multiple of 4


@pytest.mark.parametrize("axis", ["col", "both"])
@pytest.mark.parametrize("rnd", ["rne", "sr", "sr16"])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_tile_kernel_variants(dt, fmt, rnd, axis):
    dev = require_gpu()
    rng = np.random.default_rng(7)
    x = rng.standard_normal((R, C)) * np.exp2(rng.integers(-12, 12, (R, 1)) + rng.integers(-4, 4, (1, C)))
    x[rng.random((R, C)) < 0.02] = 0.0
    if fmt == "mxfp4":
        x[17, 40] = np.inf  # a non-finite block in each output direction
    xt = torch.from_numpy(x).to(dt)
    xg = xt.to(dev)
    x64 = f64(xt)
    off = OFFSET16 if rnd == "sr16" else OFFSET
    r16_t = sr_stream(rnd, C, R, SEED, off)
    r16 = sr_stream(rnd, R, C, SEED, off)
    amax = mxq.mxq_amax(xg) if fmt == "nvfp4" else None
    o = mxq.mxq_quantize(xg, fmt, axis, rnd, sr_seed=SEED, sr_offset=off, amax=amax)
    what = f"{dt} {fmt} {rnd} {axis}"
    if fmt == "mxfp4":
        ref_cc, ref_sc = mx.mxfp4_quantize_colwise(x64, r16_t=r16_t)
    else:
        ref_cc, ref_sc, st = nvfp4.nvfp4_quantize_colwise(x64, r16_t=r16_t)
        assert bits32(o.tensor_scale)[0] == np.float32(st).view(np.uint32), what + " tensor scale"
    assert_equal_bits(u8(o.codes_col), ref_cc, what + " column codes")
    assert_equal_bits(u8(o.scales_col), ref_sc, what + " column scales")
    if axis == "both":
        if fmt == "mxfp4":
            ref_cr, ref_sr = mx.mxfp4_quantize_rowwise(x64, r16=r16)
        else:
            ref_cr, ref_sr, _ = nvfp4.nvfp4_quantize_rowwise(x64, r16=r16)
        assert_equal_bits(u8(o.codes_row), ref_cr, what + " row codes")
        assert_equal_bits(u8(o.scales_row), ref_sr, what + " row scales")
