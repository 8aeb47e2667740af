"""Benchmark of the MXFP4 / NVFP4 quantise-and-convert hot path on one MI355X.

One step = one pass of every hot-path kernel over one batch of synthetic input,
the 16384 x 7168 bf16 MoE activation tensor (DeepSeek-V3 hidden size, values
0.5 * N(0,1) times a per-row log-normal magnitude):
  mxfp4_quantize      bf16 -> MXFP4 codes + E8M0 (row-wise)
  mxfp4_dequantize    MXFP4 -> bf16
  fp8_to_mxfp4        E4M3 + 1x128 fp32 scales -> MXFP4
  mxfp4_to_fp8        MXFP4 -> E4M3 + 1x128 fp32 scales
  rht_mxfp4_rowcol    random-sign H16 + MXFP4 row-wise and column-wise, one read
  nvfp4_amax          tensor amax
  nvfp4_quantize_rne  two-level NVFP4, round to nearest even
  nvfp4_quantize_sr   two-level NVFP4, Philox stochastic rounding
Throughput counts algorithmic bytes (inputs read + outputs written, as the method
defines them) over the timed steps. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E


def build_step(x, dev):
    import torch

    from mxfp4_microscaling_quantization_amd import mxq, workloads

    R, C = x.shape
    N = R * C
    q8, s128 = workloads.fp8_from_bf16(x)  # the FP8 producer's output (input of fp8_to_mxfp4)
    mask = mxq.mxq_rht_signs(4)
    u8 = torch.uint8
    qz = mxq.Quantized(torch.empty((R, C // 2), dtype=u8, device=dev), torch.empty((R, C // 32), dtype=u8, device=dev),
                       None, None, None)
    yb = torch.empty((R, C), dtype=torch.bfloat16, device=dev)
    c8 = (torch.empty((R, C // 2), dtype=u8, device=dev), torch.empty((R, C // 32), dtype=u8, device=dev))
    f8 = (torch.empty((R, C), dtype=u8, device=dev), torch.empty((R, C // 128), dtype=torch.float32, device=dev))
    rq = mxq.Quantized(torch.empty((R, C // 2), dtype=u8, device=dev), torch.empty((R, C // 32), dtype=u8, device=dev),
                       torch.empty((C, R // 2), dtype=u8, device=dev), torch.empty((C, R // 32), dtype=u8, device=dev),
                       None)
    amax = torch.empty((1,), dtype=torch.float32, device=dev)
    nq = mxq.Quantized(torch.empty((R, C // 2), dtype=u8, device=dev), torch.empty((R, C // 16), dtype=u8, device=dev),
                       None, None, torch.empty((1,), dtype=torch.float32, device=dev))
    sq = mxq.Quantized(torch.empty((R, C // 2), dtype=u8, device=dev), torch.empty((R, C // 16), dtype=u8, device=dev),
                       None, None, torch.empty((1,), dtype=torch.float32, device=dev))
    mx_b = 2 * N + N // 2 + N // 32
    f8_b = N + 4 * (N // 128) + N // 2 + N // 32
    kernels = [
        ("mxfp4_quantize", lambda: mxq.mxq_quantize(x, "mxfp4", "row", out=qz), mx_b),
        ("mxfp4_dequantize", lambda: mxq.mxq_dequantize(qz.codes_row, qz.scales_row, "mxfp4", out=yb), mx_b),
        ("fp8_to_mxfp4", lambda: mxq.mxq_fp8_to_mxfp4(q8, s128, out=c8), f8_b),
        ("mxfp4_to_fp8", lambda: mxq.mxq_mxfp4_to_fp8(c8[0], c8[1], out=f8), f8_b),
        ("rht_mxfp4_rowcol", lambda: mxq.mxq_rht_quantize(x, mask, "mxfp4", "both", out=rq),
         2 * N + 2 * (N // 2 + N // 32)),
        ("nvfp4_amax", lambda: mxq.mxq_amax(x, out=amax), 2 * N + 4),
        ("nvfp4_quantize_rne", lambda: mxq.mxq_quantize(x, "nvfp4", "row", amax=amax, out=nq),
         2 * N + N // 2 + N // 16 + 4),
        ("nvfp4_quantize_sr", lambda: mxq.mxq_quantize(x, "nvfp4", "row", "sr", sr_seed=7, amax=amax, out=sq),
         2 * N + N // 2 + N // 16 + 4),
    ]
    return kernels, (q8, s128)


def cpu_baseline(x_cpu, q8_cpu, s_cpu, rows: int):
    """The oracle (as it stands) on the first `rows` rows of the same workload."""
    import numpy as np

    from oracle import fp8 as ofp8
    from oracle import mx as omx
    from oracle import nvfp4 as onv
    from oracle import philox as oph
    from oracle import rht as orht

    xs = x_cpu[:rows].float().double().numpy()
    q8 = q8_cpu[:rows].numpy()
    s = s_cpu[:rows].numpy().view(np.uint32)
    R, C = xs.shape
    N = R * C
    mask = orht.sign_mask_from_seed(4)
    t0 = time.perf_counter()
    c, e = omx.mxfp4_quantize_rowwise(xs)
    omx.mxfp4_dequantize(c, e, "bf16")
    c8, e8 = ofp8.fp8_to_mxfp4(q8, s)
    ofp8.mxfp4_to_fp8(c8, e8)
    omx.mxfp4_quantize_rowwise(orht.rht_rowwise(xs, mask))
    omx.mxfp4_quantize_rowwise(orht.rht_rowwise(xs.T.copy(), mask))
    A = onv.tensor_amax(xs)
    onv.nvfp4_quantize_rowwise(xs, amax=A)
    onv.nvfp4_quantize_rowwise(xs, amax=A, r16=oph.tensor_r16(R, C, seed=7))
    dt = time.perf_counter() - t0
    step_bytes = (2 * (2 * N + N // 2 + N // 32) + 2 * (N + 4 * (N // 128) + N // 2 + N // 32)
                  + 2 * N + 2 * (N // 2 + N // 32) + 2 * N + 2 * (2 * N + N // 2 + N // 16))
    return step_bytes / dt / 1e9, dt


# Roofline peaks of one MI355X: HBM3E bandwidth, and the vector ALU rate for 32-bit
# integer/fp32 operations without packing (256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz).
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# Stochastic rounding is bound by its Philox4x32-10 stream, not by HBM. Algorithmic
# operations per element: Philox (10 rounds of 2 32x32->64 multiplies and 4 XORs per
# 4 words = 15), then scaling, grid floor, threshold compare and select (4).
SR_OPS_PER_ELEMENT = 19
ALU_BOUND = {"nvfp4_quantize_sr"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
SOURCES = ("include/mxq.h", "mxfp4_microscaling_quantization_amd/csrc")


def source_digest() -> str:
    """SHA-256 over the library sources: PMC traffic is reported only for the kernel
    version the counters were taken on."""
    import hashlib

    h = hashlib.sha256()
    paths = []
    for rel in SOURCES:
        p = os.path.join(ROOT, rel)
        if os.path.isdir(p):
            paths += sorted(os.path.join(p, f) for f in os.listdir(p) if f.endswith((".hip", ".h")))
        else:
            paths.append(p)
    for p in paths:
        h.update(os.path.relpath(p, ROOT).encode())
        h.update(open(p, "rb").read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed PMC summary, or None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    t = json.load(open(TRAFFIC_FILE))
    if t.get("source_sha256") != source_digest():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100, help="untimed steps (also bring the clocks up)")
    ap.add_argument("--kernel-reps", type=int, default=20, help="back-to-back launches per kernel for its duration")
    ap.add_argument("--cpu-rows", type=int, default=1024, help="rows of the oracle sample (0: skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one MI355X: the quantisation kernels need no collectives and this "
              "build runs on a single GPU; --gpus must be 1", file=sys.stderr)
        return 2

    import torch

    from mxfp4_microscaling_quantization_amd import mxq, workloads

    mxq.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    R, C = 16384, 7168
    x_cpu = workloads.moe_activations(R, C, 2)
    x = x_cpu.to(dev)
    kernels, (q8, s128) = build_step(x, dev)
    step_bytes = sum(b for _, _, b in kernels)

    for _ in range(args.warmup):
        for _, fn, _ in kernels:
            fn()
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps, bracketed by events on torch's current stream.
    E = torch.cuda.Event
    start, stop = E(enable_timing=True), E(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        for _, fn, _ in kernels:
            fn()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(stop)
    ms_per_step = gpu_ms / args.steps
    value = step_bytes * args.steps / (gpu_ms / 1e3) / 1e9
    print(f"[bench] {args.steps} steps: {gpu_ms:.3f} ms on the stream ({wall * 1e3:.3f} ms wall), "
          f"{step_bytes / 1e6:.1f} MB per step", file=sys.stderr, flush=True)

    # Per-kernel average launch duration: `kernel_reps` back-to-back launches of one
    # kernel between two events on the stream the kernels run on, so the events' own
    # cost is spread over the launches. (Inside the step a kernel also absorbs the
    # write-back of its predecessor's output; the step time above includes that.)
    per = {}
    for name, fn, b in kernels:
        fn()
        s0, s1 = E(enable_timing=True), E(enable_timing=True)
        s0.record()
        for _ in range(args.kernel_reps):
            fn()
        s1.record()
        torch.cuda.synchronize()
        us = s0.elapsed_time(s1) * 1e3 / args.kernel_reps
        gbs = b / (us * 1e-6) / 1e9
        per[name] = {"us": round(us, 3), "bytes": b, "GB_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        print(f"[bench] {name:20s} {us:9.2f} us  {gbs:8.1f} GB/s  {100 * gbs / HBM_PEAK_GBS:5.1f}% of 8 TB/s",
              file=sys.stderr, flush=True)
    # reference: a device-to-device copy of 1 GiB (read + write bytes)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = E(enable_timing=True), E(enable_timing=True)
    c0.record()
    for _ in range(10):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) * 10 / (c0.elapsed_time(c1) / 1e3) / 1e9
    del src, dst
    print(f"[bench] torch D2D copy of 1 GiB: {copy_gbs:.1f} GB/s", file=sys.stderr, flush=True)

    dom = max(per, key=lambda k: per[k]["us"])
    d = per[dom]
    traffic = measured_traffic(dom)
    if dom in ALU_BOUND:
        ops = SR_OPS_PER_ELEMENT * R * C
        tops = ops / (d["us"] * 1e-6) / 1e12
        roof = {"kernel": dom, "bound": "alu", "achieved": round(tops, 2), "peak": round(VALU_PEAK_TOPS, 2),
                "unit": "Tops/s", "frac": round(tops / VALU_PEAK_TOPS, 4), "traffic": traffic,
                "ops_per_launch": ops, "ops_per_element": SR_OPS_PER_ELEMENT, "avg_launch_us": d["us"],
                "hbm_GB_s": d["GB_s"], "hbm_frac": d["frac_hbm_peak"], "bytes_per_launch": d["bytes"]}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": d["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": d["frac_hbm_peak"], "traffic": traffic, "bytes_per_launch": d["bytes"],
                "avg_launch_us": d["us"]}

    cpu = None
    if args.cpu_rows > 0:
        cv, dt = cpu_baseline(x_cpu, q8.cpu(), s128.cpu(), args.cpu_rows)
        cpu = {"value": round(cv, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"all eight kernels' oracle counterparts on the first {args.cpu_rows} rows "
                         f"({args.cpu_rows}x{C}) of the same tensor, {dt:.1f} s, single-threaded numpy"}
        print(f"[bench] oracle sample: {cv:.4f} GB/s in {dt:.1f} s", file=sys.stderr, flush=True)

    line = {
        "metric": "quantize/convert GB/s (in+out bytes) and % of MI355X HBM peak, per kernel",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mxfp4_rowwise_16384x7168_moe: 16384x7168 bf16 MoE activations, "
                               "all eight quantise/convert kernels per step",
                   "rows": R, "cols": C, "elements_per_step": R * C, "bytes_per_step": step_bytes},
        "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "copy_reference_GB_s": round(copy_gbs, 1),
        "per_kernel": per,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
