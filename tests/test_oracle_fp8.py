"""Pins of the oracle's FP8 <-> MXFP4 conversions against torch's E4M3 codec,
exhaustive code x exponent-shift sweeps, and the losslessness condition."""
import numpy as np
import torch

from oracle import formats as F
from oracle import fp8, mx


def torch_fp8_values(q8, s):
    v = torch.from_numpy(q8).view(torch.float8_e4m3fn).to(torch.float64)
    R, C = q8.shape
    return (v.reshape(R, C // 128, 128) * torch.from_numpy(s).double()[..., None]).reshape(R, C).numpy()


def test_fp8_values_match_torch_decode():
    rng = np.random.default_rng(0)
    q8 = rng.integers(0, 256, (8, 256)).astype(np.uint8)
    q8[q8 & 0x7F == 0x7F] = 0x01  # no NaN here
    s = np.exp2(rng.integers(-20, 20, (8, 2))).astype(np.float32)
    ours = fp8.fp8_values(q8, s.view(np.uint32))
    np.testing.assert_array_equal(ours, torch_fp8_values(q8, s))


def test_fp8_to_mxfp4_equals_unfused_chain():
    # FP8 -> bf16 (exact) -> MXFP4 must give the same bits as the direct route
    rng = np.random.default_rng(1)
    x = torch.from_numpy((rng.standard_normal((64, 512)) * np.exp(rng.uniform(-3, 3, (64, 1)))).astype(np.float32))
    g = x.reshape(64, 4, 128)
    k = torch.ceil(torch.log2(g.abs().amax(-1) / 448.0))
    s = torch.exp2(k)
    q8 = (g / s[..., None]).to(torch.float8_e4m3fn).view(torch.uint8).reshape(64, 512).numpy()
    s32 = s.float().numpy()
    bf = torch.from_numpy(torch_fp8_values(q8, s32)).to(torch.bfloat16)
    assert torch.equal(bf.double(), torch.from_numpy(torch_fp8_values(q8, s32)))  # exact in bf16
    p_ref, s_ref = mx.mxfp4_quantize_rowwise(bf.double().numpy())
    p, e = fp8.fp8_to_mxfp4(q8, s32.view(np.uint32))
    np.testing.assert_array_equal(p, p_ref)
    np.testing.assert_array_equal(e, s_ref)


def test_fp8_to_mxfp4_all_codes_all_block_maxima():
    # every E4M3 code appears in a block whose maximum is every E4M3 magnitude
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]
    rows = []
    for amax_code in range(1, 127):
        blk = np.zeros(128, dtype=np.uint8)
        pick = codes[(codes & 0x7F) <= amax_code]
        blk[:min(127, len(pick))] = pick[:127]
        blk[127] = amax_code
        rows.append(blk)
    q8 = np.stack(rows)
    for sexp in (-126, -3, 0, 7, 120):
        s = np.full((q8.shape[0], 1), 2.0 ** sexp, dtype=np.float32)
        p, e = fp8.fp8_to_mxfp4(q8, s.view(np.uint32))
        vals = torch_fp8_values(q8, s)
        amax = np.abs(vals.reshape(-1, 4, 32)).max(-1)
        with np.errstate(divide="ignore", invalid="ignore"):
            expect_e = np.clip(np.floor(np.log2(amax)).astype(np.int64) - 2, -127, 127)
        expect_e = np.where(amax == 0, -127, expect_e)
        np.testing.assert_array_equal(e.astype(np.int64) - 127, expect_e)
        y = np.abs(vals.reshape(-1, 4, 32)) * np.exp2(-expect_e)[..., None]
        got = mx.unpack_nibbles(p).reshape(-1, 4, 32) & 7
        np.testing.assert_array_equal(got, F.e2m1_round_nearest_even(y))


def test_fp8_nan_and_scale_exponent_field():
    q8 = np.zeros((2, 128), dtype=np.uint8)
    q8[0, 40] = 0x7F  # E4M3 NaN in block 1
    q8[1, :] = 0x38   # 1.0
    s = np.array([[1.0], [np.float32(1.5)]], dtype=np.float32)  # 1.5: exponent field of 1.0
    p, e = fp8.fp8_to_mxfp4(q8, s.view(np.uint32))
    assert e[0].tolist() == [0, 255, 0, 0]      # zero blocks clamp to byte 0; NaN block 0xFF
    assert (p[0] == 0).all()
    assert e[1].tolist() == [125] * 4           # only the exponent field of 1.5 is read
    assert (mx.unpack_nibbles(p[1:]) == 6).all()  # 1.0 / 2^-2 = 4.0 -> code 6
    s_inf = np.array([[np.inf]], dtype=np.float32)
    p, e = fp8.fp8_to_mxfp4(q8[1:], s_inf.view(np.uint32))
    assert e.tolist() == [[255] * 4] and (p == 0).all()


def mx_group(codes16, bytes4):
    """One 128-group: the code pattern repeated over 4 blocks of 32, 4 scale bytes."""
    codes = np.resize(np.asarray(codes16, dtype=np.uint8), 128)
    return mx.pack_nibbles(codes[None, :]), np.asarray(bytes4, dtype=np.uint8)[None, :]


def test_mxfp4_to_fp8_exhaustive_codes_and_shifts():
    # all 16 codes in a block whose exponent is S - d, next to a block at S
    for S in (0, 1, 9, 127, 200, 254):
        for d in range(0, S + 1):
            packed, scales = mx_group(np.arange(16), [S, S - d, S - d, S - d])
            q8, s32 = fp8.mxfp4_to_fp8(packed, scales)
            assert s32[0, 0] == np.float32(2.0 ** (S - 127)).view(np.uint32)
            v = F.e2m1_decode(np.arange(16))
            t = v * 2.0 ** (-d)
            ref = torch.from_numpy(t.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            np.testing.assert_array_equal(q8[0, 32:48], ref)
            np.testing.assert_array_equal(q8[0, 0:16], torch.from_numpy(v.astype(np.float32)).to(
                torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_mxfp4_to_fp8_lossless_within_spread_8():
    rng = np.random.default_rng(4)
    R, C = 64, 1024
    codes = rng.integers(0, 16, (R, C)).astype(np.uint8)
    packed = mx.pack_nibbles(codes)
    base = rng.integers(20, 230, (R, C // 128, 1))
    scales = (base + rng.integers(-8, 1, (R, C // 128, 4))).reshape(R, C // 32).astype(np.uint8)
    q8, s32 = fp8.mxfp4_to_fp8(packed, scales)
    assert (np.abs(scales.reshape(R, -1, 4).astype(int).max(-1) - scales.reshape(R, -1, 4).min(-1)) <= 8).all()
    dq_fp8 = torch_fp8_values(q8, s32.view(np.float32))
    dq_mx = mx.mxfp4_dequantize_values(packed, scales)
    np.testing.assert_array_equal(dq_fp8, dq_mx)
    np.testing.assert_array_equal(np.signbit(dq_fp8), np.signbit(dq_mx))


def test_mxfp4_to_fp8_lossy_beyond_spread_8_rounds_to_nearest():
    packed, scales = mx_group([1, 2, 3, 9], [100, 91, 100, 100])  # d = 9 for block 1
    q8, _ = fp8.mxfp4_to_fp8(packed, scales)
    # 0.5 * 2^-9 = 2^-10: a tie between 0 and 2^-9 -> 0; 1.0 * 2^-9 -> 0x01; 1.5*2^-9 -> tie -> 2^-8 (0x02)
    assert q8[0, 32:36].tolist() == [0x00, 0x01, 0x02, 0x80]


def test_mxfp4_to_fp8_nan_group():
    packed, scales = mx_group(np.arange(16), [10, 255, 10, 10])
    q8, s32 = fp8.mxfp4_to_fp8(packed, scales)
    assert (q8 == 0x7F).all() and s32[0, 0] == 0x7FC00000
    packed, scales = mx_group(np.arange(16), [0, 0, 0, 0])
    q8, s32 = fp8.mxfp4_to_fp8(packed, scales)
    assert s32[0, 0] == 0x00400000  # 2^-127 is an fp32 subnormal
