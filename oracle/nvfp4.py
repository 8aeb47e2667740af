"""NVFP4 two-level quantisation: 16-element blocks, E4M3 block scale, fp32 tensor
scale; round-to-nearest-even or stochastic rounding.
TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What the pages fix ([NVFP4] section 2A "Le Format NVFP4"): blocks of 16 elements,
E2M1 elements, an E4M3 scale per block, and an fp32 scale for the whole tensor
applied on top of the block scale. Stochastic rounding is used for gradients
([NVFP4] section 2B.4).

Readings (the pages give no formulas):
  N1 the tensor scale is s_t = RN_fp32(A / (6 * 448)) with A = max |x| over the
     tensor, so the largest block scale lands on 448, the largest E4M3 value;
     A = 0 gives s_t = 0; a NaN or Inf anywhere makes A non-finite and s_t NaN.
  N2 the block scale is s_b = RNE_E4M3(a_b / (6 * s_t)) with a_b = max |x| over the
     block, the quotient taken exactly and rounded once (ties to even, saturating
     at 448).
  N3 each element's code is the E2M1 rounding of |x| / (s_b * s_t), the quotient
     taken exactly (exact real arithmetic, one rounding), sign copied, saturating
     at 6. Blocks with s_b = 0 (and every block when s_t = 0) hold sign bits only;
     when s_t is NaN every block scale byte is 0x7F and every code 0. With a
     caller-supplied amax, a block holding NaN or Inf gets byte 0x7F and codes 0.
  N4 dequantisation returns RN(v * s_b * s_t) in the output format (one rounding
     of the exact product).
  N5 column-wise NVFP4 (blocks of 16 along rows) is the row-wise quantisation of
     the transpose with the same tensor scale.
  N6 2D scaling for weights ([NVFP4] section 2B.3, 16x16 blocks): one block scale
     per 16x16 tile, s_b = RNE_E4M3(a_b / (6 * s_t)) with a_b = max |x| over the 256
     elements, codes as in N3 with that scale. The result is stored in the 1x16
     layout (each tile's scale repeated on its 16 rows), so the transpose's
     quantisation is exactly the transpose of the codes and of the scales: the
     same quantised weights serve both passes. Round to nearest even only.

Why float64 decides every rounding here exactly: each rounding compares an exact
quotient a/b (a at most 24 significant bits, b at most 28) with a threshold of at
most 20 significant bits. When they differ, their relative distance is at least
2^-48, while float64 division is correctly rounded to 2^-53, so the float64
quotient falls on the same side of every threshold and equals it only when the
exact quotient does. For s_t the quotient A/2688 has a binary expansion that
either terminates or repeats with period 6 (2^6 = 1 mod 21), so it is never within
2^-53 of an fp32 rounding midpoint without being on it.
"""
from __future__ import annotations

import numpy as np

from .formats import (e2m1_decode, e4m3_decode, e4m3_round_nearest_even,
                      round_f64_to_bf16_bits)
from .mx import e2m1_encode_magnitude, pack_nibbles, unpack_nibbles

NV_BLOCK = 16
NV_TENSOR_DIVISOR = 6.0 * 448.0  # 2688


def tensor_amax(x: np.ndarray) -> float:
    """A = max |x| over the tensor: +Inf if an infinity is present, NaN if a NaN is."""
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0:
        return 0.0
    if np.isnan(x).any():
        return float("nan")
    return float(np.abs(x).max())


def tensor_scale(amax: float) -> np.float32:
    """N1: s_t = RN_fp32(A / 2688)."""
    if not np.isfinite(amax):
        return np.float32(np.nan)
    return np.float32(np.float64(amax) / NV_TENSOR_DIVISOR)


def nvfp4_quantize_rowwise(x: np.ndarray, amax: float | None = None,
                           r16: np.ndarray | None = None):
    """Row-wise NVFP4 of a real [R, C] matrix (C % 16 == 0).

    Returns (codes uint8 [R, C/2], E4M3 block scales uint8 [R, C/16], s_t float32).
    amax: the tensor amax to use (default: computed from x). r16: optional [R, C]
    uint16 random values for stochastic rounding (see philox.py).
    """
    x = np.asarray(x, dtype=np.float64)
    R, C = x.shape
    if C % NV_BLOCK:
        raise ValueError("columns must be a multiple of 16")
    A = tensor_amax(x) if amax is None else float(amax)
    st = tensor_scale(A)
    xb = x.reshape(R, C // NV_BLOCK, NV_BLOCK)
    if np.isnan(st):
        return (np.zeros((R, C // 2), np.uint8), np.full((R, C // NV_BLOCK), 0x7F, np.uint8), st)
    sign = (np.signbit(xb).astype(np.uint8) << 3)
    if st == 0:
        return (pack_nibbles(sign.reshape(R, C)), np.zeros((R, C // NV_BLOCK), np.uint8), st)
    st64 = np.float64(st)
    finite = np.isfinite(xb).all(axis=-1)  # only reachable with a caller-given amax
    xb = np.where(finite[..., None], xb, 0.0)
    ab = np.abs(xb).max(axis=-1)
    sb_bytes = e4m3_round_nearest_even(ab / (6.0 * st64))  # N2, saturating
    sb = e4m3_decode(sb_bytes)
    denom = sb * st64  # exact in float64
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.abs(xb) / denom[..., None]
    y = np.where(sb[..., None] > 0, y, 0.0)
    rr = None if r16 is None else np.asarray(r16).reshape(xb.shape)
    mag = e2m1_encode_magnitude(y, rr)
    codes = np.where(finite[..., None], mag | sign, 0).astype(np.uint8).reshape(R, C)
    sb_bytes = np.where(finite, sb_bytes, np.uint8(0x7F)).astype(np.uint8)
    return pack_nibbles(codes), sb_bytes, st


def nvfp4_quantize_colwise(x: np.ndarray, amax: float | None = None,
                           r16_t: np.ndarray | None = None):
    """N5: column-wise NVFP4 = row-wise NVFP4 of x.T (same tensor amax)."""
    return nvfp4_quantize_rowwise(np.asarray(x, dtype=np.float64).T, amax, r16_t)


def nvfp4_dequantize_values(packed: np.ndarray, sb_bytes: np.ndarray, st: float) -> np.ndarray:
    """Exact real values v * s_b * s_t (float64 [R, C]); NaN for NaN scales."""
    codes = unpack_nibbles(packed)
    R, C = codes.shape
    v = e2m1_decode(codes).reshape(R, C // NV_BLOCK, NV_BLOCK)
    sb = e4m3_decode(sb_bytes)[..., None]
    return (v * sb * np.float64(st)).reshape(R, C)  # 2 + 4 + 24 bits: exact


def nvfp4_dequantize(packed: np.ndarray, sb_bytes: np.ndarray, st: float, out_dtype: str = "bf16"):
    """N4: bits of RN(v * s_b * s_t) as uint16 (bf16) or uint32 (fp32)."""
    v = nvfp4_dequantize_values(packed, sb_bytes, st)
    if out_dtype == "bf16":
        return round_f64_to_bf16_bits(v)
    if out_dtype == "f32":
        with np.errstate(over="ignore", invalid="ignore"):  # overflow gives +-inf (IEEE RN)
            bits = v.astype(np.float32).view(np.uint32).copy()
        bits[np.isnan(v)] = 0x7FC00000
        return bits
    raise ValueError(out_dtype)


def nvfp4_quantize_2d(x: np.ndarray, amax: float | None = None):
    """N6: NVFP4 with 16x16 block scales of a real [R, C] matrix (R, C % 16 == 0).

    Returns (codes uint8 [R, C/2], E4M3 scales uint8 [R, C/16] in the 1x16 layout
    (equal within each 16-row group), s_t float32)."""
    x = np.asarray(x, dtype=np.float64)
    R, C = x.shape
    if R % NV_BLOCK or C % NV_BLOCK:
        raise ValueError("rows and columns must be multiples of 16")
    A = tensor_amax(x) if amax is None else float(amax)
    st = tensor_scale(A)
    if np.isnan(st):
        return (np.zeros((R, C // 2), np.uint8), np.full((R, C // NV_BLOCK), 0x7F, np.uint8), st)
    sign = (np.signbit(x).astype(np.uint8) << 3)
    if st == 0:
        return (pack_nibbles(sign), np.zeros((R, C // NV_BLOCK), np.uint8), st)
    st64 = np.float64(st)
    t = x.reshape(R // NV_BLOCK, NV_BLOCK, C // NV_BLOCK, NV_BLOCK)
    finite = np.isfinite(t).all(axis=(1, 3))              # [R/16, C/16]
    ab = np.abs(np.where(finite[:, None, :, None], t, 0.0)).max(axis=(1, 3))
    sb_bytes = e4m3_round_nearest_even(ab / (6.0 * st64))  # N2 on the 16x16 amax
    sb = e4m3_decode(sb_bytes)
    denom = np.repeat(np.repeat(sb * st64, NV_BLOCK, axis=0), NV_BLOCK, axis=1)  # [R, C]
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.abs(np.where(np.isfinite(x), x, 0.0)) / denom
    y = np.where(denom > 0, y, 0.0)
    mag = e2m1_encode_magnitude(y)
    fin = np.repeat(np.repeat(finite, NV_BLOCK, axis=0), NV_BLOCK, axis=1)
    codes = np.where(fin, mag | sign, 0).astype(np.uint8)
    sb_bytes = np.where(finite, sb_bytes, np.uint8(0x7F)).astype(np.uint8)
    return pack_nibbles(codes), np.repeat(sb_bytes, NV_BLOCK, axis=0), st
