"""16-point (randomised) Hadamard transform applied ahead of MXFP4 quantisation.
TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What the pages fix:
  * a Hadamard rotation with random sign flips spreads outliers before
    quantisation; a deterministic 16-point Hadamard (H16) applies the same rotation
    every step; both are orthogonal transforms ([MXFP4-MI355X] "Expérience
    d'investigation"; [NVFP4] section 2B.2, applied to weight-gradient inputs).

Readings:
  H1 H16 is the Sylvester matrix H[i][j] = (-1)^popcount(i & j); the transform of
     every aligned 16-element chunk along the quantisation block axis is
     y = (1/4) * H16 @ (s * x): signs first, then H, scaled by 1/4 so the transform
     is orthonormal ("transformations orthogonales").
  H2 the 16 signs s_i are given by a 16-bit mask: bit i set means s_i = -1; mask 0
     is the deterministic H16. Deriving the mask from a seed is a separate helper
     (sign_mask_from_seed; the mapping is a definition made here, pinned by the
     generator's published known-answer word for seed 0 and by rocRAND's engine).
  H3 y is kept in working precision and quantised without an intermediate bf16
     rounding; this oracle computes y in float64 (the pages fix no precision).
  H4 row-wise: chunks along columns; column-wise: chunks along rows (the transform
     of x.T, then column-wise quantisation = row-wise quantisation of the transpose).
  H5 NVFP4 with the transform (the weight-gradient recipe of [NVFP4] section 2B):
     the two-level quantisation is applied to y, so the tensor scale comes from the
     amax of y (the tensor that is quantised), taken along the quantisation axis.
"""
from __future__ import annotations

import numpy as np

from .mx import mxfp4_quantize_rowwise
from .nvfp4 import nvfp4_quantize_rowwise, tensor_amax
from .philox import philox4x32_10

RHT_N = 16


def sylvester_h16() -> np.ndarray:
    """H1: H[i][j] = (-1)^popcount(i & j), as float64 [16, 16]."""
    i = np.arange(RHT_N)[:, None]
    j = np.arange(RHT_N)[None, :]
    parity = np.vectorize(lambda v: bin(int(v)).count("1") & 1)(i & j)
    return np.where(parity == 1, -1.0, 1.0)


def signs_from_mask(mask: int) -> np.ndarray:
    """H2: 16 float64 signs from a 16-bit mask (bit i set -> -1)."""
    return np.array([-1.0 if (mask >> i) & 1 else 1.0 for i in range(RHT_N)])


def sign_mask_from_seed(seed: int) -> int:
    """Sign mask for a seed: bits 0..15 of word 0 of Philox4x32-10 with
    key = (seed low 32 bits, seed high 32 bits) and counter 0. The mapping is a
    definition made here (the pages only ask for random signs); that this code
    follows it is pinned by the first published Philox vector (seed 0 gives
    0xE8D5) and by element 0 of rocRAND's engine for other seeds."""
    w = philox4x32_10(np.zeros((1, 4), dtype=np.uint32), seed)
    return int(w[0, 0]) & 0xFFFF


def rht_rowwise(x: np.ndarray, mask: int) -> np.ndarray:
    """y = (1/4) H16 (s * x) on every aligned 16-chunk of each row, float64 [R, C]."""
    x = np.asarray(x, dtype=np.float64)
    R, C = x.shape
    if C % RHT_N:
        raise ValueError("columns must be a multiple of 16")
    h = sylvester_h16()
    s = signs_from_mask(mask)
    xc = x.reshape(R, C // RHT_N, RHT_N) * s
    y = xc @ h.T * 0.25  # y_i = 1/4 sum_j H[i][j] s_j x_j
    return y.reshape(R, C)


def rht_mxfp4_rowwise(x: np.ndarray, mask: int):
    """Row-wise MXFP4 quantisation of the row-wise transform (H3, H4)."""
    return mxfp4_quantize_rowwise(rht_rowwise(x, mask))


def rht_mxfp4_colwise(x: np.ndarray, mask: int):
    """Column-wise MXFP4 quantisation of the transform taken along rows (H4):
    row-wise quantisation of rht_rowwise(x.T)."""
    return mxfp4_quantize_rowwise(rht_rowwise(np.asarray(x, dtype=np.float64).T, mask))


def rht_amax(x: np.ndarray, mask: int, axis: str = "row") -> float:
    """H5: amax of the transform taken along rows ("row") or along columns ("col")."""
    x = np.asarray(x, dtype=np.float64)
    return tensor_amax(rht_rowwise(x if axis == "row" else x.T, mask))


def rht_nvfp4_rowwise(x: np.ndarray, mask: int, amax: float | None = None, r16=None):
    """H5: row-wise NVFP4 of the row-wise transform (amax defaults to the transform's)."""
    return nvfp4_quantize_rowwise(rht_rowwise(x, mask), amax=amax, r16=r16)


def rht_nvfp4_colwise(x: np.ndarray, mask: int, amax: float | None = None, r16_t=None):
    """H5: column-wise NVFP4 of the transform along rows of x.T (H4)."""
    return nvfp4_quantize_rowwise(rht_rowwise(np.asarray(x, dtype=np.float64).T, mask), amax=amax, r16=r16_t)
