"""Python binding of libmxq: the C entry points under the same names.

Argument marshalling only: every step of the computation runs in the HIP kernels
of libmxq.so. Inputs are torch tensors on the current GPU; outputs are allocated
here with torch (device memory only) unless passed in, and every call is enqueued
on torch's current stream. A missing library raises immediately: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxq.so")

MXQ_OK, MXQ_EINVAL, MXQ_ESHAPE, MXQ_EALIGN, MXQ_EUNSUPPORTED, MXQ_EHIP = range(6)
BF16, F32 = 0, 1
MXFP4, NVFP4, NVFP4_2D = 0, 1, 2
RNE, SR, SR16 = 0, 1, 2
ROWWISE, COLWISE, BOTH = 1, 2, 3

_FMT = {"mxfp4": MXFP4, "nvfp4": NVFP4, "nvfp4_2d": NVFP4_2D}
_AXIS = {"row": ROWWISE, "col": COLWISE, "both": BOTH}
_RND = {"rne": RNE, "sr": SR, "sr16": SR16}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libmxq.so (built in-tree by mxfp4_microscaling_quantization_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m mxfp4_microscaling_quantization_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u16, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint16, ctypes.c_uint64
    L.mxq_quantize.argtypes = [vp, i32, i64, i64, i64, i32, i32, i32, u64, u64, vp, vp, vp, vp, vp, vp, vp]
    L.mxq_rht_quantize.argtypes = [vp, i32, i64, i64, i64, i32, i32, u64, i32, u64, u64, vp, vp, vp, vp,
                                   vp, vp, vp]
    L.mxq_rht_quantize_mask.argtypes = [vp, i32, i64, i64, i64, i32, i32, u16, i32, u64, u64, vp, vp, vp,
                                        vp, vp, vp, vp]
    L.mxq_dequantize.argtypes = [vp, vp, i32, i64, i64, vp, vp, i32, vp]
    L.mxq_fp8_to_mxfp4.argtypes = [vp, vp, i64, i64, vp, vp, vp]
    L.mxq_mxfp4_to_fp8.argtypes = [vp, vp, i64, i64, vp, vp, vp]
    L.mxq_fp4_row_to_fp8_col.argtypes = [vp, vp, i64, i64, vp, i64, vp, i64, vp, i64, vp]
    L.mxq_rht_apply.argtypes = [vp, i32, i64, i64, i64, u16, vp, vp]
    L.mxq_amax.argtypes = [vp, i32, i64, i64, i64, vp, vp]
    L.mxq_rht_amax.argtypes = [vp, i32, i64, i64, i64, i32, u16, vp, vp]
    L.mxq_rht_signs.argtypes = [u64]
    L.mxq_rht_signs.restype = u16
    L.mxq_status_string.argtypes = [i32]
    L.mxq_status_string.restype = ctypes.c_char_p
    for name in ("mxq_quantize", "mxq_rht_quantize", "mxq_rht_quantize_mask", "mxq_dequantize", "mxq_fp8_to_mxfp4",
                 "mxq_mxfp4_to_fp8", "mxq_fp4_row_to_fp8_col", "mxq_rht_apply", "mxq_amax", "mxq_rht_amax"):
        getattr(L, name).restype = i32
    _lib = L
    return L


class MxqError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(mxq_status_string(status))


def mxq_status_string(status: int) -> str:
    return lib().mxq_status_string(status).decode()


def mxq_rht_signs(seed: int) -> int:
    return int(lib().mxq_rht_signs(seed))


def _check(status: int) -> None:
    if status != MXQ_OK:
        raise MxqError(status)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported input dtype {t.dtype}")


def _rows_view(x: torch.Tensor):
    if x.dim() != 2 or (x.shape[0] > 0 and x.stride(1) != 1):
        raise ValueError("expected a 2-D tensor with unit column stride")
    return x.shape[0], x.shape[1], (x.stride(0) if x.shape[0] > 0 else x.shape[1])


class Quantized(NamedTuple):
    codes_row: Optional[torch.Tensor]
    scales_row: Optional[torch.Tensor]
    codes_col: Optional[torch.Tensor]
    scales_col: Optional[torch.Tensor]
    tensor_scale: Optional[torch.Tensor]


def _alloc_outputs(x, rows, cols, fmt, axis):
    bs = 32 if fmt == MXFP4 else 16
    dev = x.device
    u8 = torch.uint8
    cr = sr = cc = sc = None
    if axis & ROWWISE:
        cr = torch.empty((rows, cols // 2), dtype=u8, device=dev)
        sr = torch.empty((rows, cols // bs), dtype=u8, device=dev)
    if axis & COLWISE:
        cc = torch.empty((cols, rows // 2), dtype=u8, device=dev)
        sc = torch.empty((cols, rows // bs), dtype=u8, device=dev)
    ts = torch.empty((1,), dtype=torch.float32, device=dev) if fmt != MXFP4 else None
    return cr, sr, cc, sc, ts


def mxq_quantize(x: torch.Tensor, fmt: str = "mxfp4", axis: str = "row", rnd: str = "rne",
                 sr_seed: int = 0, sr_offset: int = 0, amax: Optional[torch.Tensor] = None,
                 out: Optional[Quantized] = None) -> Quantized:
    """mxq_quantize: MXFP4/NVFP4 quantisation. NVFP4 takes the tensor amax (e.g. from
    mxq_amax), or computes it first when `amax` is None."""
    rows, cols, ldx = _rows_view(x)
    f, a, r = _FMT[fmt], _AXIS[axis], _RND[rnd]
    o = out if out is not None else Quantized(*_alloc_outputs(x, rows, cols, f, a))
    _check(lib().mxq_quantize(_ptr(x), _dtype_code(x), rows, cols, ldx, f, a, r, sr_seed, sr_offset,
                              _ptr(o.codes_row), _ptr(o.scales_row), _ptr(o.codes_col),
                              _ptr(o.scales_col), _ptr(amax), _ptr(o.tensor_scale), _stream()))
    return o


def mxq_rht_quantize(x: torch.Tensor, rht_seed: int, fmt: str = "mxfp4", axis: str = "row",
                     rnd: str = "rne", sr_seed: int = 0, sr_offset: int = 0,
                     amax: Optional[torch.Tensor] = None, out: Optional[Quantized] = None) -> Quantized:
    """mxq_rht_quantize: random-sign 16-point Hadamard (signs drawn from `rht_seed`,
    mxq_rht_signs) fused ahead of quantisation."""
    rows, cols, ldx = _rows_view(x)
    f, a, r = _FMT[fmt], _AXIS[axis], _RND[rnd]
    o = out if out is not None else Quantized(*_alloc_outputs(x, rows, cols, f, a))
    _check(lib().mxq_rht_quantize(_ptr(x), _dtype_code(x), rows, cols, ldx, f, a, rht_seed, r, sr_seed,
                                  sr_offset, _ptr(o.codes_row), _ptr(o.scales_row), _ptr(o.codes_col),
                                  _ptr(o.scales_col), _ptr(amax), _ptr(o.tensor_scale), _stream()))
    return o


def mxq_rht_quantize_mask(x: torch.Tensor, sign_mask: int, fmt: str = "mxfp4", axis: str = "row",
                          rnd: str = "rne", sr_seed: int = 0, sr_offset: int = 0,
                          amax: Optional[torch.Tensor] = None, out: Optional[Quantized] = None) -> Quantized:
    """mxq_rht_quantize_mask: as mxq_rht_quantize with the sign mask given directly
    (bit i -> s_i = -1; 0 = the deterministic H16)."""
    rows, cols, ldx = _rows_view(x)
    f, a, r = _FMT[fmt], _AXIS[axis], _RND[rnd]
    o = out if out is not None else Quantized(*_alloc_outputs(x, rows, cols, f, a))
    _check(lib().mxq_rht_quantize_mask(_ptr(x), _dtype_code(x), rows, cols, ldx, f, a, sign_mask, r, sr_seed,
                                       sr_offset, _ptr(o.codes_row), _ptr(o.scales_row), _ptr(o.codes_col),
                                       _ptr(o.scales_col), _ptr(amax), _ptr(o.tensor_scale), _stream()))
    return o


def mxq_dequantize(codes: torch.Tensor, scales: torch.Tensor, fmt: str = "mxfp4",
                   tensor_scale: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mxq_dequantize: codes [R, C/2] + scales -> [R, C] in bf16 or fp32."""
    rows, cols = codes.shape[0], codes.shape[1] * 2
    y = out if out is not None else torch.empty((rows, cols), dtype=out_dtype, device=codes.device)
    _check(lib().mxq_dequantize(_ptr(codes), _ptr(scales), _FMT[fmt], rows, cols, _ptr(tensor_scale),
                                _ptr(y), _dtype_code(y), _stream()))
    return y


def mxq_fp8_to_mxfp4(q8: torch.Tensor, s128: torch.Tensor, out=None):
    """mxq_fp8_to_mxfp4: E4M3 [R, C] (uint8 view) + fp32 [R, C/128] -> (codes, e8m0)."""
    rows, cols = q8.shape
    if out is None:
        out = (torch.empty((rows, cols // 2), dtype=torch.uint8, device=q8.device),
               torch.empty((rows, cols // 32), dtype=torch.uint8, device=q8.device))
    _check(lib().mxq_fp8_to_mxfp4(_ptr(q8), _ptr(s128), rows, cols, _ptr(out[0]), _ptr(out[1]), _stream()))
    return out


def mxq_mxfp4_to_fp8(codes: torch.Tensor, e8m0: torch.Tensor, out=None):
    """mxq_mxfp4_to_fp8: (codes [R, C/2], e8m0 [R, C/32]) -> (E4M3 [R, C] uint8, fp32 [R, C/128])."""
    rows, cols = codes.shape[0], codes.shape[1] * 2
    if out is None:
        out = (torch.empty((rows, cols), dtype=torch.uint8, device=codes.device),
               torch.empty((rows, cols // 128), dtype=torch.float32, device=codes.device))
    _check(lib().mxq_mxfp4_to_fp8(_ptr(codes), _ptr(e8m0), rows, cols, _ptr(out[0]), _ptr(out[1]), _stream()))
    return out


def fp8_col_scale_slots(rows: int, n_experts: int) -> int:
    """Scale entries per output row that suffice for any split of `rows` into experts."""
    return (rows + 127 * n_experts) // 128


def mxq_fp4_row_to_fp8_col(codes: torch.Tensor, e8m0: torch.Tensor, offsets: torch.Tensor, out=None):
    """mxq_fp4_row_to_fp8_col: MXFP4 rows of tokens grouped by expert (device int64
    offsets [E+1]) -> (E4M3 of X^T [C, R] uint8, fp32 scales [C, S]), one scale per
    128-token group of an expert; `out` = (q8 [C, ld_q8], scales [C, ld_s])."""
    rows, cols = codes.shape[0], codes.shape[1] * 2
    n_experts = offsets.numel() - 1
    if out is None:
        ld_q8 = (rows + 15) // 16 * 16
        out = (torch.empty((cols, ld_q8), dtype=torch.uint8, device=codes.device),
               torch.empty((cols, fp8_col_scale_slots(rows, n_experts)), dtype=torch.float32,
                           device=codes.device))
    q8, s = out
    _check(lib().mxq_fp4_row_to_fp8_col(_ptr(codes), _ptr(e8m0), rows, cols, _ptr(offsets), n_experts,
                                        _ptr(q8), q8.stride(0), _ptr(s), s.stride(0), _stream()))
    return q8[:, :rows], s


def mxq_rht_apply(x: torch.Tensor, sign_mask: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mxq_rht_apply: y = (1/4) H16 (s * x) on every 16-chunk of each row, fp32."""
    rows, cols, ldx = _rows_view(x)
    y = out if out is not None else torch.empty((rows, cols), dtype=torch.float32, device=x.device)
    _check(lib().mxq_rht_apply(_ptr(x), _dtype_code(x), rows, cols, ldx, sign_mask, _ptr(y), _stream()))
    return y


def mxq_amax(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mxq_amax: max |x| over the tensor as a device fp32[1] (NaN/Inf propagate)."""
    rows, cols, ldx = _rows_view(x)
    a = out if out is not None else torch.empty((1,), dtype=torch.float32, device=x.device)
    _check(lib().mxq_amax(_ptr(x), _dtype_code(x), rows, cols, ldx, _ptr(a), _stream()))
    return a


def mxq_rht_amax(x: torch.Tensor, sign_mask: int, axis: str = "row",
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mxq_rht_amax: max |(1/4) H16 (s * x)| with the transform along rows ("row") or
    columns ("col"), as a device fp32[1]."""
    rows, cols, ldx = _rows_view(x)
    a = out if out is not None else torch.empty((1,), dtype=torch.float32, device=x.device)
    _check(lib().mxq_rht_amax(_ptr(x), _dtype_code(x), rows, cols, ldx, _AXIS[axis], sign_mask, _ptr(a),
                              _stream()))
    return a
