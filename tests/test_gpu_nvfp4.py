"""GPU parity of the NVFP4 kernels (tensor amax, two-level quantisation with
nearest-even and stochastic rounding, dequantisation) and of MXFP4 stochastic
rounding against the CPU oracle: bit-exact everywhere."""
import numpy as np
import pytest
import torch

from mxfp4_microscaling_quantization_amd import mxq, workloads
from oracle import formats as F
from oracle import mx, nvfp4, philox
from tests.gpu_helpers import assert_equal_bits, bits16, bits32, f64, require_gpu, sample_rows, u8

pytestmark = pytest.mark.gpu


def nv_check(xt: torch.Tensor, what: str, rnd: str = "rne", seed: int = 7, offset: int = 0):
    dev = require_gpu()
    xg = xt.to(dev)
    amax = mxq.mxq_amax(xg)
    x64 = f64(xt)
    A = nvfp4.tensor_amax(x64)
    got_a = float(amax.item())
    assert (np.isnan(A) and np.isnan(got_a)) or got_a == A, (got_a, A)
    o = mxq.mxq_quantize(xg, "nvfp4", "row", rnd, sr_seed=seed, sr_offset=offset, amax=amax)
    r16 = philox.tensor_r16(*x64.shape, seed=seed, offset=offset) if rnd == "sr" else None
    ref_c, ref_s, st = nvfp4.nvfp4_quantize_rowwise(x64, r16=r16)
    ts = bits32(o.tensor_scale)[0]
    assert ts == np.float32(st).view(np.uint32) or (np.isnan(st) and ts == 0x7FC00000), (hex(ts), st)
    assert_equal_bits(u8(o.scales_row), ref_s, what + " block scales")
    assert_equal_bits(u8(o.codes_row), ref_c, what + " codes")
    for dt, conv, name in ((torch.bfloat16, bits16, "bf16"), (torch.float32, bits32, "f32")):
        y = mxq.mxq_dequantize(o.codes_row, o.scales_row, "nvfp4", tensor_scale=o.tensor_scale, out_dtype=dt)
        assert_equal_bits(conv(y), nvfp4.nvfp4_dequantize(ref_c, ref_s, st, name), f"{what} dequant {name}")
    return o


@pytest.mark.parametrize("rnd", ["rne", "sr"])
def test_nvfp4_random(rnd):
    rng = np.random.default_rng(0)
    x = rng.standard_normal((96, 512)) * np.exp(rng.uniform(-6, 6, (96, 1)))
    nv_check(torch.from_numpy(x).to(torch.bfloat16), "random " + rnd, rnd, seed=11, offset=12345)


def test_nvfp4_exact_ties_and_scale_midpoints():
    # A = 2688 makes s_t exactly 1: element codes and block scales land on exact
    # rounding midpoints, which the kernel must decide with exact arithmetic
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    sbs = F.E4M3_MAGNITUDES[[20, 40, 56, 64, 72, 88, 100, 110, 119, 120]]
    rows = []
    for sb in sbs:
        blk = np.zeros(16)
        blk[0] = 6 * sb
        for i, m in enumerate(mids):
            blk[1 + i] = m * sb
            blk[8 + i] = -m * sb
        rows.append(blk)
    # block maxima on E4M3 midpoints (the block scale is a tie)
    for k in (9, 30, 60, 95, 125):
        mu = (F.E4M3_MAGNITUDES[k] + F.E4M3_MAGNITUDES[k + 1]) / 2
        blk = np.zeros(16)
        blk[0] = 6 * mu
        blk[1] = 3 * mu
        rows.append(blk)
    x = np.concatenate(rows)
    x = np.concatenate([x, np.zeros((-len(x)) % 64)]).reshape(-1, 64)
    x[0, 63] = 2688.0
    xt = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(f64(xt), x)  # all values are bf16
    for rnd in ("rne", "sr"):
        nv_check(xt, "ties " + rnd, rnd)


@pytest.mark.parametrize("case", ["zeros", "nan", "inf", "tiny_fp32", "huge", "one_big_block"])
def test_nvfp4_special_tensors(case):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 64))
    dt = torch.bfloat16
    if case == "zeros":
        x[:] = 0.0
        x[3, 7] = -0.0
    elif case == "nan":
        x[5, 5] = np.nan
    elif case == "inf":
        x[1, 2] = -np.inf
    elif case == "tiny_fp32":
        x = x * 1e-40  # s_t is an fp32 subnormal
        dt = torch.float32
    elif case == "huge":
        x = x * 1e37
    elif case == "one_big_block":
        x[0, 0] = 1e30  # every other block's scale underflows E4M3
    nv_check(torch.from_numpy(x).to(dt), case)
    nv_check(torch.from_numpy(x).to(dt), case + " sr", "sr")


def test_amax_edge_cases():
    dev = require_gpu()
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=dev)
    assert float(mxq.mxq_amax(x).item()) == 0.0
    y = torch.randn(100, 64).to(torch.bfloat16)
    y[7, 9] = float("inf")
    y[8, 1] = float("nan")
    a = mxq.mxq_amax(y.to(dev))
    assert np.isnan(float(a.item()))
    z = torch.randn(300, 128, dtype=torch.float32)
    assert float(mxq.mxq_amax(z.to(dev)[::3, 8:72]).item()) == float(z[::3, 8:72].abs().max())


@pytest.mark.parametrize("rnd", ["rne", "sr"])
def test_nvfp4_32768x4096_sampled(rnd):
    dev = require_gpu()
    w = workloads.nvfp4_activations()
    xg = w.x.to(dev)
    amax = mxq.mxq_amax(xg)
    x_all = w.x.float().numpy()
    assert float(amax.item()) == float(np.abs(x_all).max())
    o = mxq.mxq_quantize(xg, "nvfp4", "row", rnd, sr_seed=w.sr_seed, sr_offset=0, amax=amax)
    rows = sample_rows(32768, 32)
    R, C = 32768, 4096
    x64 = f64(w.x[rows])
    r16 = None
    if rnd == "sr":
        n = (rows[:, None].astype(np.uint64) * np.uint64(C) + np.arange(C, dtype=np.uint64))
        r16 = philox.element_r16(n, w.sr_seed)
    ref_c, ref_s, st = nvfp4.nvfp4_quantize_rowwise(x64, amax=float(np.abs(x_all).max()), r16=r16)
    assert bits32(o.tensor_scale)[0] == np.float32(st).view(np.uint32)
    assert_equal_bits(u8(o.scales_row[rows]), ref_s, f"32768x4096 {rnd} block scales (sampled rows)")
    assert_equal_bits(u8(o.codes_row[rows]), ref_c, f"32768x4096 {rnd} codes (sampled rows)")


def test_mxfp4_stochastic_rounding_bitexact():
    dev = require_gpu()
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 1024)) * np.exp2(rng.integers(-8, 8, (64, 1)))
    xt = torch.from_numpy(x).to(torch.bfloat16)
    o = mxq.mxq_quantize(xt.to(dev), "mxfp4", "row", "sr", sr_seed=99, sr_offset=7 * 4)
    r16 = philox.tensor_r16(64, 1024, seed=99, offset=28)
    ref_c, ref_s = mx.mxfp4_quantize_rowwise(f64(xt), r16=r16)
    assert_equal_bits(u8(o.codes_row), ref_c, "mx sr codes")
    assert_equal_bits(u8(o.scales_row), ref_s, "mx sr scales")
    # column-wise SR indexes the transpose
    o = mxq.mxq_quantize(xt.to(dev), "mxfp4", "col", "sr", sr_seed=99, sr_offset=5)
    r16t = philox.tensor_r16(1024, 64, seed=99, offset=5)
    ref_c, ref_s = mx.mxfp4_quantize_colwise(f64(xt), r16_t=r16t)
    assert_equal_bits(u8(o.codes_col), ref_c, "mx sr col codes")
    assert_equal_bits(u8(o.scales_col), ref_s, "mx sr col scales")
