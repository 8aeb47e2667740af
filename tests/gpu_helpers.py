"""Helpers shared by the GPU parity tests (bit views and sampling)."""
import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bits32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int32).numpy().view(np.uint32)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy()


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a bf16/fp32 CPU or GPU tensor."""
    return t.detach().cpu().float().double().numpy()


def sample_rows(n_rows: int, k: int, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    pick = set([0, n_rows - 1]) | set(rng.choice(n_rows, min(k, n_rows), replace=False).tolist())
    return np.array(sorted(pick))


def assert_equal_bits(got: np.ndarray, ref: np.ndarray, what: str):
    if got.shape != ref.shape:
        raise AssertionError(f"{what}: shape {got.shape} != {ref.shape}")
    bad = np.argwhere(got != ref)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: got {got[i]!r} expected {ref[i]!r}")


def sr_stream(rnd: str, rows: int, cols: int, seed: int, offset: int):
    """The oracle's random values of a rounding mode for a row-major [rows, cols]
    tensor: None (nearest even), the word stream ("sr") or the halves stream ("sr16")."""
    from oracle import philox
    if rnd == "sr":
        return philox.tensor_r16(rows, cols, seed, offset)
    if rnd == "sr16":
        return philox.tensor_r16_halves(rows, cols, seed, offset)
    return None
