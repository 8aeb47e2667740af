"""GPU parity of every variant of the row-wise kernels: bf16 and fp32 input,
contiguous and strided rows, MXFP4 and NVFP4, nearest-even and stochastic rounding,
and the dequantisation of each result to bf16 and fp32, bit-exact against the
oracle. Stochastic rounding draws word n = offset + r * C + c for element (r, c)
(halves stream: half n mod 2 of word n / 2, from an offset that is a multiple of 8)."""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_equal_bits, bits16, bits32, f64, require_gpu, sr_stream, u8
from mxfp4_microscaling_quantization_amd import mxq
from oracle import mx, nvfp4

pytestmark = pytest.mark.gpu

R, C = 77, 1056  # rows not a multiple of anything; 33 MXFP4 / 66 NVFP4 blocks per row
SEED, OFFSET, OFFSET16 = 3, 999, 1000


@pytest.mark.parametrize("strided", [False, True])
@pytest.mark.parametrize("rnd", ["rne", "sr", "sr16"])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_row_kernel_variants(dt, fmt, rnd, strided):
    dev = require_gpu()
    rng = np.random.default_rng(11)
    x = rng.standard_normal((R, C)) * np.exp2(rng.integers(-20, 20, (R, 1)))
    x[rng.random((R, C)) < 0.03] = -0.0
    if fmt == "mxfp4":
        x[5, 100] = np.nan
    xt = torch.from_numpy(x).to(dt)
    if strided:  # rows of a wider tensor, at a 16-byte-aligned column offset
        big = torch.zeros((R, C + 64), dtype=dt)
        big[:, 32:32 + C] = xt
        xg = big.to(dev)[:, 32:32 + C]
    else:
        xg = xt.to(dev)
    x64 = f64(xt)
    off = OFFSET16 if rnd == "sr16" else OFFSET
    r16 = sr_stream(rnd, R, C, SEED, off)
    amax = mxq.mxq_amax(xg) if fmt == "nvfp4" else None
    o = mxq.mxq_quantize(xg, fmt, "row", rnd, sr_seed=SEED, sr_offset=off, amax=amax)
    what = f"{dt} {fmt} {rnd} strided={strided}"
    if fmt == "mxfp4":
        ref_c, ref_s = mx.mxfp4_quantize_rowwise(x64, r16=r16)
    else:
        ref_c, ref_s, st = nvfp4.nvfp4_quantize_rowwise(x64, r16=r16)
        assert bits32(o.tensor_scale)[0] == np.float32(st).view(np.uint32), what + " tensor scale"
    assert_equal_bits(u8(o.codes_row), ref_c, what + " codes")
    assert_equal_bits(u8(o.scales_row), ref_s, what + " scales")
    for odt, conv, name in ((torch.bfloat16, bits16, "bf16"), (torch.float32, bits32, "f32")):
        if fmt == "mxfp4":
            y = mxq.mxq_dequantize(o.codes_row, o.scales_row, "mxfp4", out_dtype=odt)
            ref = mx.mxfp4_dequantize(ref_c, ref_s, name)
        else:
            y = mxq.mxq_dequantize(o.codes_row, o.scales_row, "nvfp4", tensor_scale=o.tensor_scale, out_dtype=odt)
            ref = nvfp4.nvfp4_dequantize(ref_c, ref_s, float(st), name)
        assert_equal_bits(conv(y), ref, what + f" dequantised to {name}")
