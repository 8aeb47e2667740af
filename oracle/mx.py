"""MXFP4 block quantisation and dequantisation (row-wise and column-wise).
TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What the pages fix:
  * blocks of 32 elements share one E8M0 exponent; elements are E2M1
    ([HOPPER-FR] section 1; [MXFP4-MI355X] "Qu'est-ce que le MXFP4 ?");
  * the shared exponent is "the block's maximum exponent" and each element is
    rounded to the nearest representable 4-bit value ([MXFP4-MI355X], legend of the
    reconstruction formula, whose formula itself did not survive extraction);
  * two 4-bit codes are packed per byte ([HOPPER-FR] section 1, sub-byte packing).

Readings (where the pages are silent or garbled):
  R1 shared exponent E = floor(log2 amax) - 2: the block's largest element exponent
     minus the largest E2M1 exponent (2, since 6 = 1.5 * 2^2); the OCP rule.
  R2 E is clamped to the E8M0 range [-127, 127]; the stored byte is E + 127. An
     all-zero block gets E = -127 (byte 0) and codes holding only sign bits.
  R3 a block with any NaN or +-Inf element gets scale byte 0xFF and all codes 0.
  R4 ties round to the even code; magnitudes past 6 saturate to 6.
  R5 the sign bit of a code is the input's sign bit, so -0.0 and small negatives
     give code 0x8.
  R6 nibble order: byte j of a row holds element 2j in bits 0-3 and element 2j+1 in
     bits 4-7.
  R7 column-wise quantisation (blocks of 32 along rows, the layout a weight-gradient
     GEMM consumes) is defined as the row-wise quantisation of the transpose:
     codes [C, R/2], scales [C, R/32].
"""
from __future__ import annotations

import numpy as np

from .formats import (E2M1_MAGNITUDES, e2m1_decode, e2m1_round_nearest_even,
                      e8m0_value, floor_log2, round_f64_to_bf16_bits)

MX_BLOCK = 32


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., 2n] codes (0..15) -> [..., n] bytes, element 2j in the low nibble (R6)."""
    c = np.asarray(codes).astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def mx_shared_exponent(amax: np.ndarray) -> np.ndarray:
    """R1 + R2: E = clamp(floor(log2 amax) - 2, -127, 127); amax == 0 gives -127."""
    e = floor_log2(amax) - 2
    return np.clip(e, -127, 127).astype(np.int64)


def e2m1_encode_magnitude(y: np.ndarray, r16: np.ndarray | None = None) -> np.ndarray:
    """Magnitude code (0..7) for the real magnitude y >= 0.

    r16=None: round to nearest, ties to even, saturate at 6 (R4).
    r16 given (uint16 per element): stochastic rounding. A magnitude of 6 or more
    gives 6. Otherwise, with lo the largest grid value <= y and step the distance to
    the next one, y rounds up iff y > lo + step * (r16 + 1/2) / 2^16, so values on
    the grid never move and P(up) = (y - lo)/step to within 2^-17. Rounding "to one
    of the two nearest representable values with zero expected error" is all the
    pages state ([NVFP4] section 2B.4; [MXFP4-MI355X] "Expérience d'investigation");
    using the top 16 bits of a 32-bit random word and the half-step offset is the
    reading made here (it keeps the threshold exact in 24-bit arithmetic).
    Every threshold has at most 20 significant bits, so the float64 comparison is
    exact whenever y is.
    """
    y = np.asarray(y, dtype=np.float64)
    if r16 is None:
        return e2m1_round_nearest_even(y)
    g = E2M1_MAGNITUDES
    lo = np.clip(np.searchsorted(g, y, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    step = g[hi] - g[lo]
    thr = g[lo] + step * (np.asarray(r16, dtype=np.float64) + 0.5) / 65536.0
    code = np.where(y > thr, hi, lo)
    return np.where(y >= g[-1], 7, code).astype(np.uint8)


def e2m1_encode_scaled(x: np.ndarray, e: np.ndarray, r16: np.ndarray | None = None) -> np.ndarray:
    """Signed E2M1 codes of x * 2^-e (e broadcast against x); the product is exact.

    The sign bit is copied from x (R5)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.abs(x) * np.ldexp(1.0, -e)
    mag = e2m1_encode_magnitude(y, r16)
    sign = np.signbit(x).astype(np.uint8) << 3
    return (mag | sign).astype(np.uint8)


def mxfp4_quantize_rowwise(x: np.ndarray, r16: np.ndarray | None = None):
    """Row-wise MXFP4 quantisation of a real [R, C] matrix (C % 32 == 0).

    Returns (packed codes uint8 [R, C/2], E8M0 scale bytes uint8 [R, C/32]).
    x is float64 and holds the exact input values (bf16/fp32/E4M3 times a power
    of two are all exact in float64). r16: optional [R, C] uint16 random values
    for stochastic rounding (top 16 bits of each element's Philox word, see
    philox.py); None means round to nearest even.
    """
    x = np.asarray(x, dtype=np.float64)
    R, C = x.shape
    if C % MX_BLOCK:
        raise ValueError("columns must be a multiple of 32")
    xb = x.reshape(R, C // MX_BLOCK, MX_BLOCK)
    finite = np.isfinite(xb).all(axis=-1)
    amax = np.where(finite, np.abs(np.where(np.isfinite(xb), xb, 0.0)).max(axis=-1), 0.0)
    e = mx_shared_exponent(amax)
    xs = np.where(finite[..., None], xb, 0.0)
    rr = None if r16 is None else np.asarray(r16).reshape(xb.shape)
    codes = e2m1_encode_scaled(xs, e[..., None], rr)
    codes = np.where(finite[..., None], codes, 0).astype(np.uint8)
    scales = np.where(finite, e + 127, 255).astype(np.uint8)
    return pack_nibbles(codes.reshape(R, C)), scales


def mxfp4_quantize_colwise(x: np.ndarray, r16_t: np.ndarray | None = None):
    """Column-wise MXFP4 quantisation (R7): the row-wise quantisation of x.T.

    r16_t, when given, is indexed like x.T ([C, R]).
    Returns (codes [C, R/2], scales [C, R/32]).
    """
    return mxfp4_quantize_rowwise(np.asarray(x, dtype=np.float64).T, r16_t)


def mxfp4_dequantize_values(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact real values v(code) * 2^(byte-127) as float64 [R, C]; 0xFF blocks are NaN."""
    codes = unpack_nibbles(packed)
    R, C = codes.shape
    v = e2m1_decode(codes).reshape(R, C // MX_BLOCK, MX_BLOCK)
    s = e8m0_value(scales)[..., None]
    out = v * s  # exact: a 2-bit significand times a power of two
    return out.reshape(R, C)


def mxfp4_dequantize(packed: np.ndarray, scales: np.ndarray, out_dtype: str = "bf16") -> np.ndarray:
    """Dequantised output bits: uint16 bf16 patterns or uint32 fp32 patterns.

    Each output is the exact real value rounded once to the output format (IEEE
    round-to-nearest-even, overflow to infinity); for scale bytes <= 252 every value
    is exactly representable in both formats, so no rounding happens. NaN blocks
    give the canonical quiet NaN (bf16 0x7FC0, fp32 0x7FC00000).
    """
    v = mxfp4_dequantize_values(packed, scales)
    if out_dtype == "bf16":
        return round_f64_to_bf16_bits(v)
    if out_dtype == "f32":
        with np.errstate(over="ignore", invalid="ignore"):  # overflow gives +-inf (IEEE RN)
            bits = v.astype(np.float32).view(np.uint32).copy()
        bits[np.isnan(v)] = 0x7FC00000
        return bits
    raise ValueError(out_dtype)


def mxfp4_quantize_colwise_loops(x: np.ndarray):
    """Direct column-by-column statement of column-wise quantisation, written
    without the transpose identity; used only to pin R7 on small inputs."""
    x = np.asarray(x, dtype=np.float64)
    R, C = x.shape
    codes = np.zeros((C, R), dtype=np.uint8)
    scales = np.zeros((C, R // MX_BLOCK), dtype=np.uint8)
    for c in range(C):
        for b in range(R // MX_BLOCK):
            col = x[b * MX_BLOCK:(b + 1) * MX_BLOCK, c]
            if not np.isfinite(col).all():
                scales[c, b] = 255
                continue
            amax = float(np.abs(col).max())
            e = -127 if amax == 0 else max(-127, min(127, int(np.floor(np.log2(amax))) - 2))
            scales[c, b] = e + 127
            for i in range(MX_BLOCK):
                y = abs(col[i]) * 2.0 ** (-e)
                m = int(e2m1_round_nearest_even(np.array([y]))[0])
                codes[c, b * MX_BLOCK + i] = m | (8 if np.signbit(col[i]) else 0)
    return pack_nibbles(codes), scales
