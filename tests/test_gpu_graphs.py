"""The entry points under HIP graph capture (every kernel family: row-wise, strip and
tile column-wise, 16x16 NVFP4, FP8 conversions, rows -> FP8 columns): the library
launches only kernels (the amax target is cleared by a small fill kernel, not a
memset), so a caller can capture a sequence of calls once and replay it. The graph
is replayed several times with new data copied into its static inputs, with eager
work and synchronisations between the replays, and every replay is compared with
eager calls on the same data."""
import numpy as np
import pytest
import torch

from gpu_helpers import require_gpu
from mxfp4_microscaling_quantization_amd import mxq, workloads

pytestmark = pytest.mark.gpu

R, C = 512, 1024
# token offsets of four experts for the rows -> FP8 columns call (ragged, one expert
# of a single token): 1 + 2 + 1 + 2 groups of 128 tokens
EXPERTS = [0, 100, 300, 301, 512]
GROUPS = sum((b - a + 127) // 128 for a, b in zip(EXPERTS, EXPERTS[1:]))
SCALES_COL = 31  # index of the rows -> FP8 columns scales in the outputs


def calls(x, q8, s128, off):
    out = []
    o = mxq.mxq_quantize(x, "mxfp4", "row")
    mx_codes, mx_scales = o.codes_row, o.scales_row
    out += [o.codes_row, o.scales_row]
    out.append(mxq.mxq_dequantize(o.codes_row, o.scales_row, "mxfp4", out_dtype=torch.float32))
    o = mxq.mxq_rht_quantize(x, 9, "mxfp4", "both")
    out += [o.codes_row, o.scales_row, o.codes_col, o.scales_col]
    a = mxq.mxq_amax(x)
    out.append(a)  # output 7
    o = mxq.mxq_rht_quantize(x, 9, "nvfp4", "row")  # amax of the transform computed first
    out += [o.codes_row, o.scales_row, o.tensor_scale]
    o = mxq.mxq_quantize(x, "nvfp4", "both", "sr", sr_seed=5)  # tensor amax computed first
    out += [o.codes_row, o.scales_row, o.codes_col, o.scales_col, o.tensor_scale]
    for rnd in ("rne", "sr"):
        o = mxq.mxq_quantize(x, "nvfp4", "col", rnd, sr_seed=11, sr_offset=0, amax=a)
        out += [o.codes_col, o.scales_col, o.tensor_scale]
    c, e = mxq.mxq_fp8_to_mxfp4(q8, s128)
    out += [c, e]
    out += list(mxq.mxq_mxfp4_to_fp8(c, e))
    o = mxq.mxq_quantize(x, "nvfp4_2d", "both", amax=a)
    out += [o.codes_row, o.scales_row, o.codes_col, o.scales_col]
    out += list(mxq.mxq_fp4_row_to_fp8_col(mx_codes, mx_scales, off))  # outputs 30, 31
    return out


def data(seed):
    x = workloads.outlier_normal(R, C, seed)
    q8, s128 = workloads.fp8_from_bf16(workloads.moe_activations(R, C, seed))
    return x, q8, s128


def test_captured_graph_replays_match_eager_calls():
    dev = require_gpu()
    x0, q0, s0 = data(0)
    xs, qs, ss = x0.to(dev), q0.to(dev), s0.to(dev)  # the graph's static inputs
    off = torch.tensor(EXPERTS, dtype=torch.int64, device=dev)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        calls(xs, qs, ss, off)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        static_out = calls(xs, qs, ss, off)
    for seed in (1, 2, 3, 1):
        x, q8, s128 = data(seed)
        xs.copy_(x.to(dev))
        qs.copy_(q8.to(dev))
        ss.copy_(s128.to(dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = calls(x.to(dev), q8.to(dev), s128.to(dev), off)
        torch.cuda.synchronize()
        # scale slots past the expert groups are not written
        eager[SCALES_COL] = eager[SCALES_COL][:, :GROUPS]
        replayed = list(static_out)
        replayed[SCALES_COL] = replayed[SCALES_COL][:, :GROUPS]
        assert len(eager) == SCALES_COL + 1
        for k, (u, v) in enumerate(zip(replayed, eager)):
            assert torch.equal(u.view(torch.uint8), v.view(torch.uint8)), f"replay with seed {seed}: output {k}"
    assert not np.isnan(float(static_out[7].item()))
