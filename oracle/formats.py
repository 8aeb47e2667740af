"""Number formats: E2M1 (FP4 elements), E8M0 (MX block exponent), E4M3 (FP8),
bf16 and fp32 bit views. TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Definitions restated from the pages:
  * MXFP4 elements are 4-bit floats with the E2M1 encoding and blocks of 32 share
    one E8M0 exponent ([HOPPER-FR] section 1, format incompatibility bullet;
    [MXFP4-MI355X] "Qu'est-ce que le MXFP4 ?").
  * The FP8 side of the Hopper pipeline is E4M3 ([HOPPER-FR] section 1).
  * NVFP4 block scales are E4M3 instead of UE8M0 ([NVFP4] section 2A).

Bit layouts are the OCP ones (the pages name the formats, the OCP microscaling
standard is cited by [MXFP4-MI355X] "Conclusion"):
  E2M1  s e1 e0 m   exponent bias 1; e>0: 2^(e-1)*(1+m/2); e=0: 0.5*m; no Inf/NaN
  E8M0  eeeeeeee    2^(e-127); 0xFF is NaN
  E4M3  s eeee mmm  bias 7; e>0: 2^(e-7)*(1+m/8); e=0: 2^-6*m/8; S.1111.111 is NaN,
                    no Inf, max finite 448
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------- E2M1


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code, from its bit fields."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


# magnitudes of codes 0..7 (derived from the bit fields, not typed in)
E2M1_MAGNITUDES = np.array([e2m1_value(c) for c in range(8)], dtype=np.float64)
E2M1_MAX = float(E2M1_MAGNITUDES[-1])


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """Vectorised decode of 4-bit codes (any integer array) to float64 (signed, -0 kept)."""
    codes = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAGNITUDES[codes & 7]
    return np.where((codes & 8) != 0, -mag, mag)


def _nearest_even_on_grid(mag: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the grid value nearest to mag >= 0, ties to the even index.

    grid is sorted ascending and starts at 0. A magnitude beyond the last grid value
    takes the last index (nearest finite value). Decided by exact comparisons with
    the midpoints of neighbouring grid values (each midpoint is exact in float64),
    so the result is exact for every float64 input.
    """
    n = len(grid)
    lo = np.searchsorted(grid, mag, side="right") - 1  # largest grid value <= mag
    lo = np.clip(lo, 0, n - 1)
    hi = np.minimum(lo + 1, n - 1)
    mid = (grid[lo] + grid[hi]) / 2.0
    up = (hi != lo) & ((mag > mid) | ((mag == mid) & (hi % 2 == 0)))
    return np.where(up, hi, lo)


def e2m1_round_nearest_even(y: np.ndarray) -> np.ndarray:
    """Magnitude code (0..7) of the E2M1 value nearest to y >= 0, ties to the even code.

    "Round to nearest" is how the pages quantise elements ([MXFP4-MI355X]
    "Qu'est-ce que le MXFP4 ?"); the tie rule is unstated, so ties go to the code
    whose mantissa bit is 0 (IEEE round-half-even). E2M1 has no infinity, so a value
    beyond the largest magnitude takes the nearest finite value, 6 (saturation).
    """
    y = np.asarray(y, dtype=np.float64)
    if np.any(~(y >= 0)):
        raise ValueError("e2m1_round_nearest_even takes non-negative magnitudes")
    return _nearest_even_on_grid(y, E2M1_MAGNITUDES).astype(np.uint8)


# ----------------------------------------------------------------------------- E8M0


def e8m0_value(byte: np.ndarray) -> np.ndarray:
    """2^(byte-127) as float64; 0xFF decodes to NaN."""
    b = np.asarray(byte).astype(np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)


# ----------------------------------------------------------------------------- E4M3


def e4m3_value_scalar(code: int) -> float:
    """Value of an E4M3 (OCP 'fn') byte from its bit fields."""
    s = (code >> 7) & 1
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = 2.0 ** -6 * (m / 8.0) if e == 0 else 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -mag if s else mag


E4M3_TABLE = np.array([e4m3_value_scalar(c) for c in range(256)], dtype=np.float64)
# finite magnitudes, indexed by the 7-bit magnitude code 0..126
E4M3_MAGNITUDES = E4M3_TABLE[:127].copy()
E4M3_MAX = float(E4M3_MAGNITUDES[-1])


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes).astype(np.int64) & 0xFF]


def e4m3_round_nearest_even(v: np.ndarray) -> np.ndarray:
    """E4M3 byte of the finite E4M3 value nearest to v, ties to the even code.

    Sign is copied (so -0.0 gives 0x80); NaN gives 0x7F. A magnitude beyond 448
    (infinity included) takes the nearest finite value, 448: E4M3 'fn' has no
    infinity, and the NVFP4 block scale saturates.
    """
    v = np.asarray(v, dtype=np.float64)
    nan = np.isnan(v)
    mag = np.abs(np.where(nan, 0.0, v))
    code = _nearest_even_on_grid(mag, E4M3_MAGNITUDES).astype(np.int64)
    sign = (np.signbit(v) & ~nan).astype(np.int64)
    out = (code | (sign << 7)).astype(np.uint8)
    out[nan] = 0x7F
    return out


# ----------------------------------------------------------------------------- bf16 / fp32


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def f32_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)


def round_f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16 bits of RNE(v): one rounding of the (exact) float64 value to bf16.

    bf16 has 8 significant bits and fp32's exponent range (normal down to 2^-126,
    subnormal quantum 2^-133). The value is rounded to the nearest multiple of its
    quantum with ties to even (np.round), then overflow past the largest finite
    value goes to infinity as in IEEE round-to-nearest. NaN gives 0x7FC0.
    """
    v = np.asarray(v, dtype=np.float64)
    nan = np.isnan(v)
    vv = np.where(nan, 0.0, v)
    a = np.abs(vv)
    with np.errstate(divide="ignore"):
        _, e = np.frexp(a)  # a = f * 2^e, f in [0.5, 1)
    exp = np.maximum(e - 1, -126)  # floor(log2 a), clamped to the subnormal range
    quantum = np.ldexp(1.0, exp - 7)
    r = np.round(vv / quantum) * quantum
    big = np.abs(r) >= 2.0 ** 128
    r = np.where(big, np.copysign(np.inf, vv), r)
    r = np.where(np.isinf(vv), vv, r)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(nan, np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


def f64_to_f32_bits(v: np.ndarray) -> np.ndarray:
    """fp32 bits of RNE(v) (numpy's float64->float32 cast rounds once, to nearest even)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).view(np.uint32)


def floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2 a) for a > 0 (exact, from frexp); -2**30 for a == 0."""
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(divide="ignore"):
        _, e = np.frexp(a)
    return np.where(a > 0, e.astype(np.int64) - 1, np.int64(-(2 ** 30)))
