"""The C ABI from a plain C program: tests/c_caller/mxq_c_caller.c is compiled with
gcc against include/mxq.h and the HIP runtime (no PyTorch, no Python binding), reads
a seeded bf16 tensor from a file into memory from hipMalloc, quantises it to MXFP4
row- and column-wise in one call, dequantises the rows, quantises it to NVFP4 with no
amax given (the library computes the tensor amax first), and converts the MXFP4 rows
to FP8 columns per 128-token group of ragged experts; every output is compared with
the oracle bit for bit."""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

from gpu_helpers import assert_equal_bits, require_gpu
from mxfp4_microscaling_quantization_amd import workloads
from oracle import fp8, mx, nvfp4

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mxfp4_microscaling_quantization_amd")
SRC = os.path.join(ROOT, "tests", "c_caller", "mxq_c_caller.c")
ROCM = "/opt/rocm"


def build(tmp):
    lib = os.path.join(PKG, "libmxq.so")
    assert os.path.exists(lib), "libmxq.so is not built"
    cc = shutil.which("gcc") or shutil.which("cc")
    assert cc, "no C compiler"
    exe = os.path.join(tmp, "mxq_c_caller")
    subprocess.run([cc, "-std=c99", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC, "-o", exe,
                    "-L", PKG, "-lmxq", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"],
                   check=True, capture_output=True, text=True)
    return exe


# expert token offsets (ragged, one expert of a single token)
OFFSETS = {96: [0, 40, 41, 96], 1024: [0, 100, 300, 301, 1024]}


@pytest.mark.parametrize("rows,cols", [(96, 544), (1024, 4096)])
def test_c_program_matches_oracle(tmp_path, rows, cols):
    require_gpu()
    exe = build(str(tmp_path))
    x = workloads.moe_activations(rows, cols, 21).cpu().contiguous()  # bf16
    src = os.path.join(str(tmp_path), "x.bin")
    x.view(torch.int16).numpy().tofile(src)
    prefix = os.path.join(str(tmp_path), "out")
    print(f"C caller {rows}x{cols}", flush=True)
    off = OFFSETS[rows]
    r = subprocess.run([exe, str(rows), str(cols), src, prefix, *map(str, off)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    got = {k: np.fromfile(f"{prefix}.{k}", dtype=np.uint8)
           for k in ("codes_row", "scales_row", "codes_col", "scales_col")}
    deq = np.fromfile(f"{prefix}.deq_row", dtype=np.uint16)

    xf = x.float().numpy().astype(np.float64)
    ref_c, ref_s = mx.mxfp4_quantize_rowwise(xf)
    ref_cc, ref_sc = mx.mxfp4_quantize_colwise(xf)
    assert_equal_bits(got["codes_row"].reshape(rows, cols // 2), ref_c, "C caller: row codes")
    assert_equal_bits(got["scales_row"].reshape(rows, cols // 32), ref_s, "C caller: row scales")
    assert_equal_bits(got["codes_col"].reshape(cols, rows // 2), ref_cc, "C caller: column codes")
    assert_equal_bits(got["scales_col"].reshape(cols, rows // 32), ref_sc, "C caller: column scales")
    assert_equal_bits(deq.reshape(rows, cols), mx.mxfp4_dequantize(ref_c, ref_s, "bf16"), "C caller: dequantised rows")
    nv_c, nv_s, st = nvfp4.nvfp4_quantize_rowwise(xf)  # amax computed from x
    assert np.fromfile(f"{prefix}.nv_st", dtype=np.float32)[0].view(np.uint32) == np.float32(st).view(np.uint32)
    assert_equal_bits(np.fromfile(f"{prefix}.nv_scales", dtype=np.uint8).reshape(rows, cols // 16), nv_s,
                      "C caller: NVFP4 block scales (NULL amax)")
    assert_equal_bits(np.fromfile(f"{prefix}.nv_codes", dtype=np.uint8).reshape(rows, cols // 2), nv_c,
                      "C caller: NVFP4 codes (NULL amax)")
    ref_q8, ref_sb = fp8.mxfp4_rows_to_fp8_cols(ref_c, ref_s, np.array(off, dtype=np.int64))
    ld_q8, ld_s, groups = (rows + 15) // 16 * 16, (rows + 127 * (len(off) - 1)) // 128, ref_sb.shape[1]
    q8 = np.fromfile(f"{prefix}.fc_q8", dtype=np.uint8).reshape(cols, ld_q8)[:, :rows]
    sb = np.fromfile(f"{prefix}.fc_s", dtype=np.uint32).reshape(cols, ld_s)[:, :groups]
    assert_equal_bits(q8, ref_q8, "C caller: FP8 columns")
    assert_equal_bits(sb, ref_sb, "C caller: FP8 column scales")
