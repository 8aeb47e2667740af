"""Seeded synthetic inputs shaped like the workloads the pages train on.

This module holds input recipes only: no quantisation arithmetic of the library
lives here, and both the HIP path (through tests and the benchmark) and the CPU
oracle receive the same arrays from it. Every generator uses numpy's PCG64
``default_rng(seed)`` with a fixed draw order and casts fp32 to bf16 with torch
(round to nearest even).

Shapes stand in for the pages' models: hidden size 7168 with 256 routed experts
for the 671B DeepSeek-V3-like MoE of "Practical FP4 Training for Large-Scale MoE
Models on Hopper GPUs" (section 4), and hidden 4096 / FFN 14336 for the
Llama-3.1-8B pretraining of "Pretraining large language models with MXFP4 on
Native FP4 Hardware". No dataset or trained weights are used.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


def _to_bf16(x32: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)


def outlier_normal(rows: int, cols: int, seed: int) -> torch.Tensor:
    """N(0,1) with 0.1% of entries (chosen without replacement) scaled by 100; bf16."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((rows, cols), dtype=np.float32)
    n = rows * cols
    idx = rng.choice(n, n // 1000, replace=False)
    z.reshape(-1)[idx] *= np.float32(100.0)
    return _to_bf16(z)


def moe_activations(rows: int, cols: int, seed: int) -> torch.Tensor:
    """0.5 * N(0,1) times a per-row log-normal(0,1) magnitude; bf16.

    'N(0, 0.5)' is read as standard deviation 0.5."""
    rng = np.random.default_rng(seed)
    m = rng.lognormal(0.0, 1.0, rows).astype(np.float32)
    z = rng.standard_normal((rows, cols), dtype=np.float32)
    z *= np.float32(0.5)
    z *= m[:, None]
    return _to_bf16(z)


def heavy_tailed_gradients(rows: int, cols: int, seed: int) -> torch.Tensor:
    """1e-3 * (N(0,1) + Student-t(3)); bf16 (the noise scale is read as 1e-3 too)."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((rows, cols), dtype=np.float32)
    t = rng.standard_t(3, (rows, cols)).astype(np.float32)
    z += t
    z *= np.float32(1e-3)
    return _to_bf16(z)


def expert_counts(tokens: int, experts: int, seed: int, alpha: float = 0.5) -> np.ndarray:
    """Tokens per expert ~ multinomial(tokens, Dirichlet(alpha)); int64 [experts]."""
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.full(experts, alpha))
    return rng.multinomial(tokens, p).astype(np.int64)


def mxfp4_codes(rows: int, cols: int, seed: int):
    """Row-wise MXFP4 data shaped like stored MoE activations, drawn directly (no
    quantisation happens here): packed codes uint8 [R, C/2] (element 2j in the low
    nibble) and E8M0 bytes uint8 [R, C/32].

    One random byte per element: its low 4 bits pick the magnitude code 1..7 with
    weights 1, 2, 2, 3, 3, 3, 2 (roughly the codes of Gaussian blocks scaled to a
    maximum in [4, 8)), bit 4 the sign, and the element is zero when bits 5-7 are
    all clear (1/8). A block's byte is 127 plus the rounded log2 of a per-row
    log-normal(0, 1) magnitude, minus 2, plus a block jitter in {-1, 0, 1}.
    """
    rng = np.random.default_rng(seed)
    lut = np.array([1, 2, 2, 3, 3, 4, 4, 4, 5, 5, 5, 6, 6, 6, 7, 7], dtype=np.uint8)
    r = rng.integers(0, 256, (rows, cols), dtype=np.uint8)
    nib = lut[r & 15]
    nib[(r >> 5) == 0] = 0
    nib |= (r & 16) >> 1
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    row_e = np.round(rng.standard_normal((rows, 1)) / np.log(2.0)).astype(np.int64)
    jitter = rng.integers(-1, 2, (rows, cols // 32))
    e8m0 = np.clip(127 - 2 + row_e + jitter, 0, 254).astype(np.uint8)
    return torch.from_numpy(packed), torch.from_numpy(e8m0)


def fp8_from_bf16(x: torch.Tensor):
    """E4M3 codes and per-1x128 power-of-two fp32 scales of a bf16 [R, C] tensor.

    This is the FP8 producer the conversion kernels consume, not part of the
    library: per 128-group, s = 2^k with k the smallest integer such that
    max|x|/2^k <= 448 (k = 0 for an all-zero group); codes are torch's
    float8_e4m3fn cast of x/2^k (exact scaling, round to nearest even).
    Returns (q8 uint8 [R, C], s float32 [R, C/128]).
    """
    R, C = x.shape
    g = x.float().reshape(R, C // 128, 128)
    a = g.abs().amax(dim=-1)
    # smallest k with a <= 448 * 2^k
    k = torch.ceil(torch.log2(a.double() / 448.0)).to(torch.int32)
    k = torch.where(a > 0, k, torch.zeros_like(k))
    # guard the log2 rounding: step k until a/2^k <= 448 < a/2^(k-1)
    for _ in range(2):
        k = torch.where((a > 0) & (torch.ldexp(a, -k.float()) > 448.0), k + 1, k)
        k = torch.where((a > 0) & (torch.ldexp(a, -(k - 1).float()) <= 448.0), k - 1, k)
    s = torch.ldexp(torch.ones_like(a), k.float())
    q = (g / s[..., None]).to(torch.float8_e4m3fn).view(torch.uint8).reshape(R, C)
    return q, s.contiguous()


@dataclass
class Workload:
    name: str
    x: torch.Tensor | None = None          # bf16 input
    q8: torch.Tensor | None = None         # uint8 E4M3 input (FP8 configs)
    s128: torch.Tensor | None = None       # fp32 [R, C/128] scales
    offsets: np.ndarray | None = None      # expert segment offsets (rows)
    codes: torch.Tensor | None = None      # packed MXFP4 codes input
    e8m0: torch.Tensor | None = None       # E8M0 block bytes of `codes`
    rht_seed: int | None = None
    sr_seed: int | None = None


# Full-size workloads (name -> builder). Sizes are the pages' model dimensions.
def mxfp4_rowwise_small(rows: int = 1024, cols: int = 4096) -> Workload:
    return Workload("mxfp4_rowwise_1024x4096_outliers", x=outlier_normal(rows, cols, 0))


def mxfp4_rowwise_moe(rows: int = 16384, cols: int = 7168) -> Workload:
    return Workload("mxfp4_rowwise_16384x7168_moe", x=moe_activations(rows, cols, 2))


def fp8_moe_experts(rows: int = 65536, cols: int = 7168, experts: int = 256) -> Workload:
    counts = expert_counts(rows, experts, 1)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    x = moe_activations(rows, cols, 1)
    q8, s = fp8_from_bf16(x)
    return Workload("fp8_mxfp4_65536x7168_256experts", q8=q8, s128=s, offsets=offsets)


def fp8_col_experts(rows: int = 65536, cols: int = 7168, experts: int = 256) -> Workload:
    """MXFP4 token buffer of the MoE layer (the same expert split as fp8_moe_experts)
    for the rows-to-FP8-columns conversion of the weight gradient."""
    counts = expert_counts(rows, experts, 1)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    codes, e8m0 = mxfp4_codes(rows, cols, 3)
    return Workload("fp4_row_to_fp8_col_65536x7168_256experts", codes=codes, e8m0=e8m0, offsets=offsets)


def rht_gradients(rows: int = 8192, cols: int = 14336) -> Workload:
    return Workload("rht_mxfp4_rowcol_8192x14336_grads", x=heavy_tailed_gradients(rows, cols, 4),
                    rht_seed=4)


def nvfp4_activations(rows: int = 32768, cols: int = 4096) -> Workload:
    return Workload("nvfp4_32768x4096_outliers", x=outlier_normal(rows, cols, 5), sr_seed=7)
