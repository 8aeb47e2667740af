"""The boundary's calls in the forms the library's interface specifies: NVFP4 with no
amax given (the call computes the tensor amax first, in the tensor-scale slot, and
quantises from it) and the Hadamard transform drawn from a seed. Bit-exact against
the CPU oracle, and bit-identical to the explicit-amax / explicit-mask calls."""
import numpy as np
import pytest
import torch

from mxfp4_microscaling_quantization_amd import mxq, workloads
from oracle import mx, nvfp4, philox, rht
from tests.gpu_helpers import assert_equal_bits, bits32, f64, require_gpu, u8

pytestmark = pytest.mark.gpu


def st_bits(st) -> int:
    return int(np.float32(st).view(np.uint32))


@pytest.mark.parametrize("rnd", ["rne", "sr"])
@pytest.mark.parametrize("axis", ["row", "col", "both"])
def test_nvfp4_null_amax_matches_oracle(axis, rnd):
    dev = require_gpu()
    xt = workloads.outlier_normal(96, 320, 13)
    x64 = f64(xt)
    xg = xt.to(dev)
    o = mxq.mxq_quantize(xg, "nvfp4", axis, rnd, sr_seed=7, sr_offset=5)
    A = nvfp4.tensor_amax(x64)
    st = nvfp4.tensor_scale(A)
    assert bits32(o.tensor_scale)[0] == st_bits(st)
    if axis in ("row", "both"):
        r16 = philox.tensor_r16(96, 320, seed=7, offset=5) if rnd == "sr" else None
        rc, rs, _ = nvfp4.nvfp4_quantize_rowwise(x64, r16=r16)
        assert_equal_bits(u8(o.codes_row), rc, "null-amax NVFP4 row codes")
        assert_equal_bits(u8(o.scales_row), rs, "null-amax NVFP4 row scales")
    if axis in ("col", "both"):
        r16 = philox.tensor_r16(320, 96, seed=7, offset=5) if rnd == "sr" else None
        rc, rs, _ = nvfp4.nvfp4_quantize_colwise(x64, A, r16)
        assert_equal_bits(u8(o.codes_col), rc, "null-amax NVFP4 col codes")
        assert_equal_bits(u8(o.scales_col), rs, "null-amax NVFP4 col scales")
    # the same bits as the two-call form (mxq_amax, then quantise with the amax)
    o2 = mxq.mxq_quantize(xg, "nvfp4", axis, rnd, sr_seed=7, sr_offset=5, amax=mxq.mxq_amax(xg))
    for a, b in zip(o, o2):
        if a is not None:
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("case", ["zeros", "nan", "inf", "fp32_tiny"])
def test_nvfp4_null_amax_special_tensors(case):
    dev = require_gpu()
    rng = np.random.default_rng(4)
    x = rng.standard_normal((32, 64))
    dt = torch.bfloat16
    if case == "zeros":
        x[:] = 0.0
        x[1, 2] = -0.0
    elif case == "nan":
        x[5, 17] = np.nan
    elif case == "inf":
        x[9, 40] = -np.inf
    else:
        x *= 2.0 ** -140
        dt = torch.float32
    xt = torch.from_numpy(x).to(dt)
    x64 = f64(xt)
    o = mxq.mxq_quantize(xt.to(dev), "nvfp4", "row")
    rc, rs, st = nvfp4.nvfp4_quantize_rowwise(x64)
    got = bits32(o.tensor_scale)[0]
    assert got == st_bits(st) or (np.isnan(st) and got == 0x7FC00000), (hex(got), st)
    assert_equal_bits(u8(o.scales_row), rs, case + " scales")
    assert_equal_bits(u8(o.codes_row), rc, case + " codes")


def test_nvfp4_2d_null_amax():
    dev = require_gpu()
    xt = workloads.outlier_normal(128, 256, 6)
    x64 = f64(xt)
    o = mxq.mxq_quantize(xt.to(dev), "nvfp4_2d", "both")
    c, s, st = nvfp4.nvfp4_quantize_2d(x64)
    ct, sct, _ = nvfp4.nvfp4_quantize_2d(x64.T.copy())
    assert bits32(o.tensor_scale)[0] == st_bits(st)
    assert_equal_bits(u8(o.codes_row), c, "2d rows")
    assert_equal_bits(u8(o.scales_row), s, "2d row scales")
    assert_equal_bits(u8(o.codes_col), ct, "2d cols")
    assert_equal_bits(u8(o.scales_col), sct, "2d col scales")


def test_null_amax_without_tensor_scale_slot_is_rejected():
    dev = require_gpu()
    x = torch.zeros((32, 64), dtype=torch.bfloat16, device=dev)
    o = mxq.mxq_quantize(x, "nvfp4", "row", amax=mxq.mxq_amax(x))
    with pytest.raises(mxq.MxqError) as e:
        mxq.mxq_quantize(x, "nvfp4", "row", out=o._replace(tensor_scale=None))
    assert e.value.status == mxq.MXQ_EINVAL


@pytest.mark.parametrize("seed", [0, 4, 2 ** 40 + 9])
def test_rht_from_seed_equals_mask_call(seed):
    dev = require_gpu()
    xg = workloads.heavy_tailed_gradients(64, 256, 1).to(dev)
    mask = mxq.mxq_rht_signs(seed)
    assert mask == rht.sign_mask_from_seed(seed)
    for fmt, axis in (("mxfp4", "both"), ("nvfp4", "row"), ("nvfp4", "col")):
        a = mxq.mxq_rht_quantize(xg, seed, fmt, axis)
        b = mxq.mxq_rht_quantize_mask(xg, mask, fmt, axis, amax=mxq.mxq_rht_amax(xg, mask, axis) if fmt == "nvfp4" else None)
        for u, v in zip(a, b):
            if u is not None:
                assert torch.equal(u.view(torch.uint8), v.view(torch.uint8)), (fmt, axis)


@pytest.mark.parametrize("rnd", ["rne", "sr"])
def test_rht_from_seed_bitexact_on_exact_inputs(rnd):
    # small integers times 2^-3: every butterfly sum is exact in fp32, so the seeded
    # transform + quantisation is bit-exact against the oracle (the sign of an exact
    # zero aside)
    dev = require_gpu()
    rng = np.random.default_rng(12)
    x = rng.integers(-48, 49, (64, 128)) * 2.0 ** -3
    xt = torch.from_numpy(x).to(torch.bfloat16)
    seed = 2 ** 33 + 17
    mask = rht.sign_mask_from_seed(seed)
    o = mxq.mxq_rht_quantize(xt.to(dev), seed, "mxfp4", "both", rnd, sr_seed=3)
    r16 = philox.tensor_r16(64, 128, seed=3) if rnd == "sr" else None
    r16t = philox.tensor_r16(128, 64, seed=3) if rnd == "sr" else None
    y = rht.rht_rowwise(x, mask)
    yt = rht.rht_rowwise(x.T.copy(), mask)
    for got_c, got_s, yy, rr in ((o.codes_row, o.scales_row, y, r16), (o.codes_col, o.scales_col, yt, r16t)):
        rc, rs = mx.mxfp4_quantize_rowwise(yy, rr)
        assert np.array_equal(u8(got_s), rs)
        g, r = mx.unpack_nibbles(u8(got_c)), mx.unpack_nibbles(rc)
        assert np.array_equal(g & 7, r & 7)
        nz = yy != 0
        assert np.array_equal((g >> 3)[nz], (r >> 3)[nz])
    # NVFP4 with the amax of the transform computed by the call itself
    for axis in ("row", "col"):
        on = mxq.mxq_rht_quantize(xt.to(dev), seed, "nvfp4", axis, rnd, sr_seed=3)
        a = rht.rht_amax(x, mask, axis)
        assert bits32(on.tensor_scale)[0] == st_bits(nvfp4.tensor_scale(a))
        if axis == "row":
            rc, rs, _ = rht.rht_nvfp4_rowwise(x, mask, amax=a, r16=r16)
            gc, gs, yy = u8(on.codes_row), u8(on.scales_row), y
        else:
            rc, rs, _ = rht.rht_nvfp4_colwise(x, mask, amax=a, r16_t=r16t)
            gc, gs, yy = u8(on.codes_col), u8(on.scales_col), yt
        assert np.array_equal(gs, rs), axis
        g, r = mx.unpack_nibbles(gc), mx.unpack_nibbles(rc)
        assert np.array_equal(g & 7, r & 7), axis
        nz = yy != 0
        assert np.array_equal((g >> 3)[nz], (r >> 3)[nz]), axis
