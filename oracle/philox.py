"""Philox4x32-10 counter-based random numbers.
TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages only say that stochastic rounding draws random numbers ([NVFP4]
section 2B.4); the generator is Philox4x32 with 10 rounds as published by
Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
(SC'11), restated here from its definition:
  state: four 32-bit counter words (c0, c1, c2, c3) and two key words (k0, k1);
  one round: (hi0, lo0) = 64-bit product M0 * c0, (hi1, lo1) = M1 * c2, then
     (c0, c1, c2, c3) <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0);
  the key is bumped by the Weyl constants (W0, W1) between rounds; ten rounds.
  Constants: M0 = 0xD2511F53, M1 = 0xCD9E8D57, W0 = 0x9E3779B9, W1 = 0xBB67AE85.

Element stream (the reading of "per-element offset = linear index"): element n of
a tensor uses the 32-bit word (n mod 4) of Philox(counter = (floor(n/4) low 32
bits, floor(n/4) high 32 bits, 0, 0), key = (seed low 32, seed high 32)); n is
the caller's base offset plus the element's row-major index in the tensor being
quantised. Stochastic rounding uses the top 16 bits of that word.

Opt-in cheaper stream (16-bit halves; a definition made here, not in the pages):
element n uses the 16-bit half (n mod 2) -- the low half for even n -- of word
((n mod 8) div 2) of Philox(counter = (floor(n/8) low, floor(n/8) high, 0, 0), same
key), so one generator call serves eight consecutive elements. Equivalently, it is
half (n mod 2) of word (n div 2) of the default element stream. It trades the
per-element 32-bit word for a 16-bit value, which is all the rounding rule reads.
"""
from __future__ import annotations

import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counters: np.ndarray, seed: int) -> np.ndarray:
    """Philox4x32-10 of counters [N, 4] (uint32) under the 64-bit seed -> [N, 4] uint32."""
    c = np.asarray(counters, dtype=np.uint32).astype(np.uint64)
    c0, c1, c2, c3 = c[:, 0], c[:, 1], c[:, 2], c[:, 3]
    k0 = seed & 0xFFFFFFFF
    k1 = (seed >> 32) & 0xFFFFFFFF
    for rnd in range(10):
        p0 = M0 * c0  # < 2^64, exact in uint64
        p1 = M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0)
        k0 = (k0 + W0) & 0xFFFFFFFF
        k1 = (k1 + W1) & 0xFFFFFFFF
    return np.stack([c0, c1, c2, c3], axis=1).astype(np.uint32)


def element_words(n: np.ndarray, seed: int) -> np.ndarray:
    """32-bit random word of each element index n (uint64 array, any shape)."""
    n = np.asarray(n, dtype=np.uint64)
    flat = n.reshape(-1)
    ctr = flat >> np.uint64(2)
    counters = np.zeros((flat.size, 4), dtype=np.uint32)
    counters[:, 0] = (ctr & MASK32).astype(np.uint32)
    counters[:, 1] = (ctr >> np.uint64(32)).astype(np.uint32)
    w = philox4x32_10(counters, seed)
    sel = (flat & np.uint64(3)).astype(np.int64)
    return w[np.arange(flat.size), sel].reshape(n.shape)


def element_r16(n: np.ndarray, seed: int) -> np.ndarray:
    """Top 16 bits of each element's word (the stochastic-rounding input)."""
    return (element_words(n, seed) >> np.uint32(16)).astype(np.uint16)


def tensor_r16(rows: int, cols: int, seed: int, offset: int = 0) -> np.ndarray:
    """r16 for every element of a row-major [rows, cols] tensor, n = offset + r*cols + c."""
    n = np.uint64(offset) + np.arange(rows * cols, dtype=np.uint64)
    return element_r16(n, seed).reshape(rows, cols)


def element_r16_halves(n: np.ndarray, seed: int) -> np.ndarray:
    """The 16-bit value of each element index n in the opt-in halves stream."""
    n = np.asarray(n, dtype=np.uint64)
    flat = n.reshape(-1)
    ctr = flat >> np.uint64(3)
    counters = np.zeros((flat.size, 4), dtype=np.uint32)
    counters[:, 0] = (ctr & MASK32).astype(np.uint32)
    counters[:, 1] = (ctr >> np.uint64(32)).astype(np.uint32)
    w = philox4x32_10(counters, seed)
    word = w[np.arange(flat.size), ((flat & np.uint64(7)) >> np.uint64(1)).astype(np.int64)]
    half = (flat & np.uint64(1)).astype(np.uint32)
    return ((word >> (np.uint32(16) * half)) & np.uint32(0xFFFF)).astype(np.uint16).reshape(n.shape)


def tensor_r16_halves(rows: int, cols: int, seed: int, offset: int = 0) -> np.ndarray:
    """Halves-stream values for a row-major [rows, cols] tensor, n = offset + r*cols + c."""
    n = np.uint64(offset) + np.arange(rows * cols, dtype=np.uint64)
    return element_r16_halves(n, seed).reshape(rows, cols)
