"""GPU parity of the FP8 (E4M3, 1x128 scale) <-> MXFP4 conversions against the CPU
oracle: bit-exact codes, exponents, FP8 bytes and fp32 scales; per-expert ragged
segments give the same bits as one call."""
import numpy as np
import pytest
import torch

from mxfp4_microscaling_quantization_amd import mxq, workloads
from oracle import fp8, mx
from tests.gpu_helpers import assert_equal_bits, bits32, require_gpu, sample_rows, u8

pytestmark = pytest.mark.gpu


def run_both(q8: np.ndarray, s: np.ndarray, what: str):
    dev = require_gpu()
    qg = torch.from_numpy(q8).to(dev)
    sg = torch.from_numpy(s.astype(np.float32)).to(dev)
    codes, e8 = mxq.mxq_fp8_to_mxfp4(qg, sg)
    ref_c, ref_e = fp8.fp8_to_mxfp4(q8, s.astype(np.float32).view(np.uint32))
    assert_equal_bits(u8(e8), ref_e, what + " e8m0")
    assert_equal_bits(u8(codes), ref_c, what + " codes")
    q8b, s128 = mxq.mxq_mxfp4_to_fp8(codes, e8)
    ref_q, ref_s = fp8.mxfp4_to_fp8(ref_c, ref_e)
    assert_equal_bits(u8(q8b), ref_q, what + " fp8 bytes")
    assert_equal_bits(bits32(s128), ref_s, what + " fp8 scales")


def test_all_e4m3_codes_and_scale_exponents():
    rng = np.random.default_rng(0)
    R, C = 256, 512
    q8 = rng.integers(0, 256, (R, C)).astype(np.uint8)
    q8[rng.random((R, C)) < 0.001] = 0x7F  # a few NaNs
    # blocks whose maximum walks through every magnitude code
    q8[:, ::32] = (np.arange(R * C // 32) % 127).astype(np.uint8).reshape(R, C // 32)
    sexp = rng.integers(-140, 140, (R, C // 128))
    s = np.ldexp(1.0, np.clip(sexp, -126, 127)).astype(np.float32)
    s[0, 0] = np.float32(np.inf)       # exponent field 255: NaN group
    s[1, 1] = np.float32(1.5)          # only the exponent field is read
    s[2, 2] = np.float32(2.0 ** -140)  # subnormal: exponent field 0
    run_both(q8, s, "random codes")


def test_zero_and_negative_zero_groups():
    q8 = np.zeros((4, 256), dtype=np.uint8)
    q8[1] = 0x80
    q8[2, 7] = 0x01
    q8[3, 100] = 0xFE
    s = np.ones((4, 2), dtype=np.float32)
    run_both(q8, s, "zeros")


def test_mxfp4_to_fp8_random_exponent_spreads():
    dev = require_gpu()
    rng = np.random.default_rng(3)
    R, C = 128, 1024
    codes = mx.pack_nibbles(rng.integers(0, 16, (R, C)).astype(np.uint8))
    base = rng.integers(0, 255, (R, C // 128, 1))
    e = np.clip(base - rng.integers(0, 20, (R, C // 128, 4)), 0, 254).reshape(R, C // 32).astype(np.uint8)
    e[5, 9] = 255
    q8, s128 = mxq.mxq_mxfp4_to_fp8(torch.from_numpy(codes).to(dev), torch.from_numpy(e).to(dev))
    ref_q, ref_s = fp8.mxfp4_to_fp8(codes, e)
    assert_equal_bits(u8(q8), ref_q, "spread fp8 bytes")
    assert_equal_bits(bits32(s128), ref_s, "spread scales")


def test_small_moe_buffer_bitexact():
    w = workloads.fp8_moe_experts(rows=2048, cols=7168, experts=16)
    run_both(u8(w.q8), w.s128.numpy(), "moe 2048x7168")


def test_moe_65536x7168_256_experts_sampled_and_segments():
    dev = require_gpu()
    w = workloads.fp8_moe_experts()
    qg, sg = w.q8.to(dev), w.s128.to(dev)
    codes, e8 = mxq.mxq_fp8_to_mxfp4(qg, sg)
    q8b, s128 = mxq.mxq_mxfp4_to_fp8(codes, e8)
    rows = sample_rows(qg.shape[0], 40)
    q8_np = u8(w.q8[rows])
    s_np = w.s128[rows].numpy().view(np.uint32)
    ref_c, ref_e = fp8.fp8_to_mxfp4(q8_np, s_np)
    assert_equal_bits(u8(codes[rows]), ref_c, "moe codes (sampled rows)")
    assert_equal_bits(u8(e8[rows]), ref_e, "moe e8m0 (sampled rows)")
    ref_q, ref_s = fp8.mxfp4_to_fp8(ref_c, ref_e)
    assert_equal_bits(u8(q8b[rows]), ref_q, "moe fp8 (sampled rows)")
    assert_equal_bits(bits32(s128[rows]), ref_s, "moe fp8 scales (sampled rows)")
    # ragged per-expert segments (some empty): one call per segment == one call
    off = w.offsets
    assert (np.diff(off) == 0).any()
    c2 = torch.empty_like(codes)
    e2 = torch.empty_like(e8)
    q2 = torch.empty_like(q8b)
    s2 = torch.empty_like(s128)
    for a, b in zip(off[:-1], off[1:]):
        a, b = int(a), int(b)
        mxq.mxq_fp8_to_mxfp4(qg[a:b], sg[a:b], out=(c2[a:b], e2[a:b]))
        mxq.mxq_mxfp4_to_fp8(codes[a:b], e8[a:b], out=(q2[a:b], s2[a:b]))
    assert torch.equal(c2, codes) and torch.equal(e2, e8)
    assert torch.equal(q2, q8b) and torch.equal(s2.view(torch.int32), s128.view(torch.int32))
    # a property over the whole buffer: the FP8 round trip is exact wherever the
    # four block exponents of a group lie within 8 of each other
    ev = e8.view(-1, 4).to(torch.int32)
    tight = (ev.amax(1) - ev.amin(1)) <= 8
    back_c, back_e = mxq.mxq_fp8_to_mxfp4(q8b, s128)
    same = (back_c.view(-1, 64) == codes.view(-1, 64)).all(1) & (back_e.view(-1, 4) == e8.view(-1, 4)).all(1)
    assert bool(same[tight].all())
