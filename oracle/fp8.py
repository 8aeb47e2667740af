"""FP8 (E4M3 with one fp32 scale per 1x128 group) <-> MXFP4 conversions.
TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What the pages fix ([HOPPER-FR] section 2B "Algorithmes de conversion directe";
[HOPPER-ES] section 2, "Conversión Directa FP4 a FP8" and "Manejo de Subnormales"):
  * the FP8 side is E4M3 with one scale per 128 consecutive elements of a row,
    the FP4 side MXFP4 with blocks of 32;
  * FP8 -> FP4 is a direct quantisation with no BF16 intermediate;
  * FP4 -> FP8 remaps sign/exponent/mantissa fields without intermediate float
    arithmetic; the single FP8 scale of a 128-group is the largest of its four
    32-block scales, and each element's exponent is adjusted so the represented
    value is preserved; subnormal results get their implicit bit materialised.

Readings:
  F1 the fp32 scale s of an FP8 group is read through its exponent field only:
     s_eff = 2^(expfield(s) - 127) (so a power of two is used as is); an exponent
     field of 255 (Inf/NaN) makes every block of the group NaN (scale byte 0xFF).
  F2 FP8 -> MXFP4 is defined as MXFP4 quantisation of the exact values
     e4m3(q) * s_eff (the direct algorithm reaches exactly this result); an E4M3
     NaN makes its 32-block NaN; the MX exponent clamps to [-127, 127].
  F3 MXFP4 -> FP8: S = max of the group's four E8M0 bytes; each element becomes the
     E4M3 value nearest to v(code) * 2^(E_j - S) (ties to even; subnormals kept;
     sign and -0 kept); the output scale is the fp32 value 2^(S - 127) (2^-127 is
     the fp32 subnormal 0x00400000). A group with any 0xFF byte gets scale NaN
     (0x7FC00000) and all codes 0x7F. Exact whenever the four exponents of the
     blocks with nonzero codes are within 8 of each other.
  F4 MXFP4 rows -> FP8 columns, the fused dequantise / transpose / requantise step
     that feeds the weight gradient of each expert ([HOPPER-FR] section 2C,
     "Fusion d'opérateurs" and "Gestion des tenseurs ragged"; [HOPPER-ES] section
     2, "Kernels CUDA Especializados", FP4RowToFP8Col). The input's rows are tokens
     grouped by expert (offsets o_0 = 0 <= ... <= o_E = R, no padding). The output
     is X^T as FP8: row c holds column c of X, the experts' token segments side by
     side. Along each row, every expert's tokens are cut into groups of 128
     starting at the expert's first token (the last group keeps the remainder);
     each group has one fp32 scale. The pages do not give the scale rule for this
     direction; it is read as the rule of the FP8 tensors consumed elsewhere here:
     s = 2^k with k the smallest integer such that max|x| / 2^k <= 448 (k = 0 for
     an all-zero group), codes the nearest-even E4M3 of x / s (exact quotient,
     subnormals kept, sign and -0 kept). A group that meets a NaN block (E8M0
     0xFF) gets scale NaN (0x7FC00000) and all codes 0x7F. Scales of group g of
     expert e sit at index sum_{e' < e} ceil(n_e' / 128) + g of the row.
"""
from __future__ import annotations

import numpy as np

from .formats import e2m1_decode, e4m3_decode, e4m3_round_nearest_even, floor_log2
from .mx import MX_BLOCK, mxfp4_dequantize_values, mxfp4_quantize_rowwise, unpack_nibbles

FP8_GROUP = 128


def fp8_scale_exponent(s_bits: np.ndarray) -> np.ndarray:
    """F1: exponent field of fp32 scale bit patterns (uint32) -> int64 (0..255)."""
    return ((np.asarray(s_bits, dtype=np.uint32) >> 23) & 0xFF).astype(np.int64)


def fp8_values(q8: np.ndarray, s_bits: np.ndarray) -> np.ndarray:
    """Exact real values e4m3(q8) * s_eff of an FP8 tensor [R, C] with group scales
    [R, C/128] given as fp32 bit patterns (F1). NaN where the element or the group
    scale is NaN/Inf."""
    q8 = np.asarray(q8, dtype=np.uint8)
    R, C = q8.shape
    ef = fp8_scale_exponent(s_bits)
    v = e4m3_decode(q8).reshape(R, C // FP8_GROUP, FP8_GROUP)
    s = np.where(ef == 255, np.nan, np.ldexp(1.0, ef - 127))[..., None]
    return (v * s).reshape(R, C)


def fp8_to_mxfp4(q8: np.ndarray, s_bits: np.ndarray):
    """F2: FP8 E4M3 [R, C] + fp32 group scales [R, C/128] -> (codes [R, C/2], E8M0 [R, C/32])."""
    C = np.asarray(q8).shape[1]
    if C % FP8_GROUP:
        raise ValueError("columns must be a multiple of 128")
    return mxfp4_quantize_rowwise(fp8_values(q8, s_bits))


def mxfp4_to_fp8(packed: np.ndarray, scales: np.ndarray):
    """F3: MXFP4 (codes [R, C/2], E8M0 [R, C/32]) -> (E4M3 [R, C], fp32 scale bits [R, C/128])."""
    codes = unpack_nibbles(packed)
    R, C = codes.shape
    if C % FP8_GROUP:
        raise ValueError("columns must be a multiple of 128")
    e = np.asarray(scales).astype(np.int64).reshape(R, C // FP8_GROUP, FP8_GROUP // MX_BLOCK)
    nan_group = (e == 255).any(axis=-1)
    S = e.max(axis=-1)
    shift = (e - S[..., None])  # <= 0
    v = e2m1_decode(codes).reshape(R, C // FP8_GROUP, FP8_GROUP // MX_BLOCK, MX_BLOCK)
    t = v * np.ldexp(1.0, shift)[..., None]  # exact real target values
    q8 = e4m3_round_nearest_even(t).reshape(R, C // FP8_GROUP, FP8_GROUP)
    q8 = np.where(nan_group[..., None], np.uint8(0x7F), q8).astype(np.uint8)
    with np.errstate(over="ignore"):  # S = 255 overflows; replaced by NaN below
        s = np.ldexp(1.0, S - 127).astype(np.float32).view(np.uint32)
    s = np.where(nan_group, np.uint32(0x7FC00000), s).astype(np.uint32)
    return q8.reshape(R, C), s


def fp8_group_exponent(amax: np.ndarray) -> np.ndarray:
    """F4: smallest integer k with amax / 2^k <= 448 (k = 0 where amax == 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    k = np.where(amax > 0, floor_log2(np.where(amax > 0, amax, 1.0)) - 8, 0).astype(np.int64)
    pos = amax > 0
    # walk k to the smallest value that keeps the group within the E4M3 range
    for _ in range(4):
        k = np.where(pos & (amax > 448.0 * np.ldexp(1.0, k)), k + 1, k)
        k = np.where(pos & (amax <= 448.0 * np.ldexp(1.0, k - 1)), k - 1, k)
    return k


def expert_group_offsets(offsets: np.ndarray) -> np.ndarray:
    """F4: index of each expert's first 128-token group: prefix sums of ceil(n_e / 128)."""
    o = np.asarray(offsets, dtype=np.int64)
    n = o[1:] - o[:-1]
    if (n < 0).any() or o[0] != 0:
        raise ValueError("offsets must start at 0 and be nondecreasing")
    return np.concatenate([[0], np.cumsum((n + FP8_GROUP - 1) // FP8_GROUP)]).astype(np.int64)


def mxfp4_rows_to_fp8_cols(packed: np.ndarray, scales: np.ndarray, offsets: np.ndarray):
    """F4: MXFP4 rows (codes [R, C/2], E8M0 [R, C/32]) of tokens grouped by expert
    (offsets [E+1]) -> (E4M3 [C, R], fp32 scale bits [C, G]) with G the total number
    of 128-token groups."""
    x = mxfp4_dequantize_values(packed, scales)  # exact; NaN blocks are NaN
    R, C = x.shape
    o = np.asarray(offsets, dtype=np.int64)
    if o[-1] != R:
        raise ValueError("the last offset must be the number of rows")
    gofs = expert_group_offsets(o)
    q8 = np.zeros((C, R), np.uint8)
    s = np.zeros((C, int(gofs[-1])), np.uint32)
    xt = x.T
    for e in range(len(o) - 1):
        for g, t0 in enumerate(range(int(o[e]), int(o[e + 1]), FP8_GROUP)):
            t1 = min(t0 + FP8_GROUP, int(o[e + 1]))
            seg = xt[:, t0:t1]                        # [C, n]: one group per row
            nan = np.isnan(seg).any(axis=1)
            amax = np.abs(np.where(np.isnan(seg), 0.0, seg)).max(axis=1)
            k = fp8_group_exponent(amax)
            codes = e4m3_round_nearest_even(seg / np.ldexp(1.0, k)[:, None])
            q8[:, t0:t1] = np.where(nan[:, None], np.uint8(0x7F), codes)
            sb = np.ldexp(1.0, k).astype(np.float32).view(np.uint32)
            s[:, gofs[e] + g] = np.where(nan, np.uint32(0x7FC00000), sb)
    return q8, s


def fp8_dequantize_values(q8: np.ndarray, s_bits: np.ndarray) -> np.ndarray:
    """Exact real values of an FP8 tensor with group scales (same as fp8_values)."""
    return fp8_values(q8, s_bits)
