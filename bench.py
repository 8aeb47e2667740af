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
defines them) over the timed steps. After the step, the rows beyond it are timed
at their own shapes (16x16-scaled NVFP4, RHT + NVFP4 column-wise, MXFP4 stochastic
rounding, MXFP4 rows -> FP8 columns of the 256-expert token buffer) together with
the fused-vs-unfused ablation of the FP8 <-> MXFP4 conversions. Prints one JSON
line.
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


def build_step(x, dev, sets: int = 3):
    """The eight kernels of one step, over `sets` independent buffer sets.

    Within a set every kernel reads its own copy of its input (identical data), and
    steps rotate through the sets, so no launch finds its input in the 256 MB MALL or
    the L2: every input byte comes from HBM (a set is about 2.2 GB). Returns
    (kernels, fp8 input) where kernels[i] = (name, fn(set), algorithmic bytes)."""
    import torch

    from mxfp4_microscaling_quantization_amd import mxq, workloads

    R, C = x.shape
    N = R * C
    q8_0, s128_0 = workloads.fp8_from_bf16(x.cpu())
    mask = mxq.mxq_rht_signs(4)
    u8 = torch.uint8

    def e(*shape, dtype=u8):
        return torch.empty(shape, dtype=dtype, device=dev)

    S = []
    for _ in range(sets):
        st = {"xa": x.clone(), "xr": x.clone(), "xm": x.clone(), "xn": x.clone(), "xs": x.clone(),
              "q8": q8_0.to(dev), "s128": s128_0.to(dev)}
        st["deq_in"] = mxq.mxq_quantize(st["xa"], "mxfp4", "row")
        st["f8_in"] = mxq.mxq_fp8_to_mxfp4(st["q8"], st["s128"])
        st["qz"] = mxq.Quantized(e(R, C // 2), e(R, C // 32), None, None, None)
        st["yb"] = e(R, C, dtype=torch.bfloat16)
        st["c8"] = (e(R, C // 2), e(R, C // 32))
        st["f8"] = (e(R, C), e(R, C // 128, dtype=torch.float32))
        st["rq"] = mxq.Quantized(e(R, C // 2), e(R, C // 32), e(C, R // 2), e(C, R // 32), None)
        st["amax"] = e(1, dtype=torch.float32)
        st["nq"] = mxq.Quantized(e(R, C // 2), e(R, C // 16), None, None, e(1, dtype=torch.float32))
        st["sq"] = mxq.Quantized(e(R, C // 2), e(R, C // 16), None, None, e(1, dtype=torch.float32))
        S.append(st)
    torch.cuda.synchronize()
    mx_b = 2 * N + N // 2 + N // 32
    f8_b = N + 4 * (N // 128) + N // 2 + N // 32
    nv_b = 2 * N + N // 2 + N // 16 + 4
    kernels = [
        ("mxfp4_quantize", lambda k: mxq.mxq_quantize(S[k]["xa"], "mxfp4", "row", out=S[k]["qz"]), mx_b),
        ("mxfp4_dequantize", lambda k: mxq.mxq_dequantize(S[k]["deq_in"].codes_row, S[k]["deq_in"].scales_row,
                                                          "mxfp4", out=S[k]["yb"]), mx_b),
        ("fp8_to_mxfp4", lambda k: mxq.mxq_fp8_to_mxfp4(S[k]["q8"], S[k]["s128"], out=S[k]["c8"]), f8_b),
        ("mxfp4_to_fp8", lambda k: mxq.mxq_mxfp4_to_fp8(S[k]["f8_in"][0], S[k]["f8_in"][1], out=S[k]["f8"]), f8_b),
        ("rht_mxfp4_rowcol", lambda k: mxq.mxq_rht_quantize(S[k]["xr"], mask, "mxfp4", "both", out=S[k]["rq"]),
         2 * N + 2 * (N // 2 + N // 32)),
        ("nvfp4_amax", lambda k: mxq.mxq_amax(S[k]["xm"], out=S[k]["amax"]), 2 * N + 4),
        ("nvfp4_quantize_rne", lambda k: mxq.mxq_quantize(S[k]["xn"], "nvfp4", "row", amax=S[k]["amax"],
                                                          out=S[k]["nq"]), nv_b),
        ("nvfp4_quantize_sr", lambda k: mxq.mxq_quantize(S[k]["xs"], "nvfp4", "row", "sr", sr_seed=7,
                                                         amax=S[k]["amax"], out=S[k]["sq"]), nv_b),
    ]
    return kernels, (q8_0, s128_0)


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


def config_report(dev, reps: int = 30) -> list:
    """Each configuration of the pages' workloads at its own shape: per-kernel average
    duration over `reps` back-to-back launches (after a warm-up), GB/s, elements/s and
    % of the HBM peak. Launches rotate through copies of the buffers whose total
    exceeds the 256 MB MALL, so every input is read from HBM."""
    import torch

    from mxfp4_microscaling_quantization_amd import mxq, workloads

    E = torch.cuda.Event

    def timed(fn, n):
        for k in range(5):
            fn(k % n)
        torch.cuda.synchronize()
        a, b = E(enable_timing=True), E(enable_timing=True)
        a.record()
        for k in range(reps):
            fn(k % n)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    def graph_timed(fn, n):
        # the same launches captured once in a HIP graph: the device time per launch
        # without the host's per-call launch cost
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for k in range(3):
                fn(k % n)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(reps):
                fn(k % n)
        g.replay()
        torch.cuda.synchronize()
        a, b = E(enable_timing=True), E(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    out = []

    def row(cfg, name, fn, n, nbytes, elems, graph=False):
        warm()
        us = graph_timed(fn, n) if graph else timed(fn, n)
        r = {"config": cfg, "kernel": name, "us": round(us, 3), "bytes": nbytes, "GB_s": round(nbytes / us / 1e3, 1),
             "elements_per_s": round(elems / (us * 1e-6), 1), "frac_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
             "buffer_sets": n}
        print("[config] " + json.dumps(r), file=sys.stderr, flush=True)
        out.append(r)

    def copies(t, n):
        return [t.to(dev) for _ in range(n)]

    # the inputs are generated on the host while the GPU idles: bring its clocks up
    # again before each configuration is timed
    w = workloads.mxfp4_rowwise_moe().x.to(dev)

    def warm():
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.3:
            mxq.mxq_quantize(w, "mxfp4", "row", "sr", sr_seed=1)
            torch.cuda.synchronize()
    for cfg, n, wl in ((1, 64, workloads.mxfp4_rowwise_small()), (2, 3, workloads.mxfp4_rowwise_moe())):
        xs = copies(wl.x, n)
        R, C = wl.x.shape
        N = R * C
        qs = [mxq.mxq_quantize(x, "mxfp4", "row") for x in xs]
        ys = [torch.empty_like(x) for x in xs]
        b = 2 * N + N // 2 + N // 32
        qfn = lambda k: mxq.mxq_quantize(xs[k], "mxfp4", "row", out=qs[k])  # noqa: E731
        dfn = lambda k: mxq.mxq_dequantize(qs[k].codes_row, qs[k].scales_row, "mxfp4", out=ys[k])  # noqa: E731
        row(cfg, "mxfp4_quantize", qfn, n, b, N)
        row(cfg, "mxfp4_dequantize", dfn, n, b, N)
        if cfg == 1:  # a 10.6 MB tensor: the per-call launch cost dominates eager launches
            row(cfg, "mxfp4_quantize (HIP graph)", qfn, n, b, N, graph=True)
            row(cfg, "mxfp4_dequantize (HIP graph)", dfn, n, b, N, graph=True)
        del xs, qs, ys
    n = 2
    wl = workloads.fp8_moe_experts()
    q8s, s128s = copies(wl.q8, n), copies(wl.s128, n)
    N = wl.q8.numel()
    c8s = [mxq.mxq_fp8_to_mxfp4(q8s[k], s128s[k]) for k in range(n)]
    f8s = [mxq.mxq_mxfp4_to_fp8(*c8s[k]) for k in range(n)]
    b = N + 4 * (N // 128) + N // 2 + N // 32
    row(3, "fp8_to_mxfp4", lambda k: mxq.mxq_fp8_to_mxfp4(q8s[k], s128s[k], out=c8s[k]), n, b, N)
    row(3, "mxfp4_to_fp8", lambda k: mxq.mxq_mxfp4_to_fp8(c8s[k][0], c8s[k][1], out=f8s[k]), n, b, N)
    del q8s, s128s, c8s, f8s, wl
    n = 3
    wl = workloads.rht_gradients()
    xs = copies(wl.x, n)
    N = wl.x.numel()
    mask = mxq.mxq_rht_signs(wl.rht_seed)
    os_ = [mxq.mxq_rht_quantize(x, mask, "mxfp4", "both") for x in xs]
    b = 2 * N + 2 * (N // 2 + N // 32)
    row(4, "rht_mxfp4_rowcol", lambda k: mxq.mxq_rht_quantize(xs[k], mask, "mxfp4", "both", out=os_[k]), n, b, N)
    row(4, "mxfp4_rowcol (no RHT)", lambda k: mxq.mxq_quantize(xs[k], "mxfp4", "both", out=os_[k]), n, b, N)
    row(4, "rht_mxfp4_col", lambda k: mxq.mxq_rht_quantize(xs[k], mask, "mxfp4", "col", out=os_[k]), n,
        b - N // 2 - N // 32, N)
    del xs, os_, wl
    wl = workloads.nvfp4_activations()
    xs = copies(wl.x, n)
    N = wl.x.numel()
    amax = [mxq.mxq_amax(x) for x in xs]
    os_ = [mxq.mxq_quantize(x, "nvfp4", "row", amax=a) for x, a in zip(xs, amax)]
    b = 2 * N + N // 2 + N // 16 + 4
    row(5, "nvfp4_amax", lambda k: mxq.mxq_amax(xs[k], out=amax[k]), n, 2 * N + 4, N)
    row(5, "nvfp4_quantize_rne", lambda k: mxq.mxq_quantize(xs[k], "nvfp4", "row", amax=amax[k], out=os_[k]), n, b, N)
    row(5, "nvfp4_quantize_sr", lambda k: mxq.mxq_quantize(xs[k], "nvfp4", "row", "sr", sr_seed=wl.sr_seed,
                                                            amax=amax[k], out=os_[k]), n, b, N)
    del w
    return out


def next_rows(dev, x, reps: int = 20) -> tuple[dict, dict]:
    """The rows beyond the eight-kernel step, each at its own shape with rotating
    input copies (no input found in a cache): 16x16-scaled NVFP4 of the MoE tensor
    (both outputs), RHT + NVFP4 column-wise (the weight-gradient recipe), MXFP4 with
    stochastic rounding, the fused MXFP4-rows -> FP8-columns conversion of the
    65536 x 7168 token buffer of 256 experts; and the fused-vs-unfused ablation of
    the two FP8 <-> MXFP4 conversions against op-by-op chains through bf16 (torch
    casts for the FP8 side), with a bit comparison of the two routes."""
    import numpy as np
    import torch

    from mxfp4_microscaling_quantization_amd import mxq, workloads

    E = torch.cuda.Event
    R, C = x.shape
    N = R * C

    def timed(fn, n):
        for k in range(n):
            fn(k)
        torch.cuda.synchronize()
        a, b = E(enable_timing=True), E(enable_timing=True)
        a.record()
        for k in range(reps):
            fn(k % n)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    rows = {}

    def row(name, fn, n, nbytes, note):
        us = timed(fn, n)
        gbs = nbytes / (us * 1e-6) / 1e9
        rows[name] = {"us": round(us, 3), "bytes": nbytes, "GB_s": round(gbs, 1),
                      "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "workload": note}
        print(f"[next] {name:24s} {us:9.2f} us  {gbs:8.1f} GB/s  {100 * gbs / HBM_PEAK_GBS:5.1f}%",
              file=sys.stderr, flush=True)
        return us

    n = 3
    xs = [x.clone() for _ in range(n)]
    am = [mxq.mxq_amax(v) for v in xs]
    q2 = [mxq.mxq_quantize(v, "nvfp4_2d", "both", amax=a) for v, a in zip(xs, am)]
    row("nvfp4_2d_rowcol", lambda k: mxq.mxq_quantize(xs[k], "nvfp4_2d", "both", amax=am[k], out=q2[k]), n,
        2 * N + 2 * (N // 2 + N // 16) + 4, f"{R}x{C} bf16 MoE tensor, 16x16 block scales, both outputs")
    del q2
    mask = mxq.mxq_rht_signs(4)
    ra = [mxq.mxq_rht_amax(v, mask, "col") for v in xs]
    rq = [mxq.mxq_rht_quantize(v, mask, "nvfp4", "col", amax=a) for v, a in zip(xs, ra)]
    row("rht_nvfp4_col", lambda k: mxq.mxq_rht_quantize(xs[k], mask, "nvfp4", "col", amax=ra[k], out=rq[k]), n,
        2 * N + N // 2 + N // 16 + 4, f"{R}x{C} bf16, H16 along rows, column-wise NVFP4")
    row("rht_amax_col", lambda k: mxq.mxq_rht_amax(xs[k], mask, "col", out=ra[k]), n, 2 * N + 4,
        f"{R}x{C} bf16, amax of the column-wise transform")
    del rq
    sq = [mxq.mxq_quantize(v, "mxfp4", "row") for v in xs]
    row("mxfp4_quantize_sr", lambda k: mxq.mxq_quantize(xs[k], "mxfp4", "row", "sr", sr_seed=7, out=sq[k]), n,
        2 * N + N // 2 + N // 32, f"{R}x{C} bf16, Philox stochastic rounding")

    # ---- fused vs unfused (the pages' kernel-level claim, measured here)
    abl = {}
    q8c, s128c = workloads.fp8_from_bf16(x.cpu())
    q8 = [q8c.to(dev) for _ in range(n)]
    s128 = [s128c.to(dev) for _ in range(n)]
    f_out = [mxq.mxq_fp8_to_mxfp4(q8[k], s128[k]) for k in range(n)]
    yb = [torch.empty((R, C), dtype=torch.bfloat16, device=dev) for _ in range(n)]

    def fp8_unfused(k):
        v = q8[k].view(torch.float8_e4m3fn).to(torch.bfloat16).view(R, C // 128, 128)
        torch.mul(v, s128[k].to(torch.bfloat16)[..., None], out=yb[k].view(R, C // 128, 128))
        return mxq.mxq_quantize(yb[k], "mxfp4", "row", out=sq[k])

    fb = N + 4 * (N // 128) + N // 2 + N // 32
    t_f = row("fp8_to_mxfp4 (fused)", lambda k: mxq.mxq_fp8_to_mxfp4(q8[k], s128[k], out=f_out[k]), n, fb,
              f"{R}x{C} E4M3 + 1x128 scales")
    t_u = row("fp8_to_mxfp4 (unfused)", fp8_unfused, n, fb, "torch E4M3->bf16 cast and scaling, then mxq_quantize")
    u = fp8_unfused(0)
    torch.cuda.synchronize()
    same = bool(torch.equal(u.codes_row, f_out[0][0]) and torch.equal(u.scales_row, f_out[0][1]))
    # the bytes an ideal unfused chain must move: FP8 in, bf16 out, bf16 in, MXFP4 out
    ideal = (N + 4 * (N // 128) + 2 * N + 2 * N + N // 2 + N // 32) / fb
    abl["fp8_to_mxfp4"] = {"fused_us": round(t_f, 3), "unfused_us": round(t_u, 3),
                           "speedup": round(t_u / t_f, 3), "same_bits": same,
                           "unfused_to_fused_bytes": round(ideal, 3)}
    b_out = [mxq.mxq_mxfp4_to_fp8(*f_out[k]) for k in range(n)]
    q8o = [torch.empty((R, C), dtype=torch.uint8, device=dev) for _ in range(n)]

    def mx_unfused(k):
        mxq.mxq_dequantize(f_out[k][0], f_out[k][1], "mxfp4", out=yb[k])
        smax = f_out[k][1].view(R, C // 128, 4).amax(-1).to(torch.int32)
        sc = torch.ldexp(torch.ones((), device=dev), (smax - 127).float())
        q = torch.div(yb[k].view(R, C // 128, 128).float(), sc[..., None]).to(torch.float8_e4m3fn)
        q8o[k].copy_(q.view(torch.uint8).view(R, C))
        return q8o[k], sc

    t_f = row("mxfp4_to_fp8 (fused)", lambda k: mxq.mxq_mxfp4_to_fp8(*f_out[k], out=b_out[k]), n, fb,
              f"{R}x{C} MXFP4 -> E4M3 + 1x128 scales")
    t_u = row("mxfp4_to_fp8 (unfused)", mx_unfused, n, fb, "mxq_dequantize to bf16, then torch scaling and E4M3 cast")
    uq, us_ = mx_unfused(0)
    torch.cuda.synchronize()
    same = bool(torch.equal(uq, b_out[0][0]) and torch.equal(us_.float(), b_out[0][1]))
    abl["mxfp4_to_fp8"] = {"fused_us": round(t_f, 3), "unfused_us": round(t_u, 3),
                           "speedup": round(t_u / t_f, 3), "same_bits": same,
                           "unfused_to_fused_bytes": round(ideal, 3)}
    del xs, am, ra, sq, q8, s128, f_out, yb, b_out, q8o
    torch.cuda.empty_cache()

    # ---- MXFP4 rows -> FP8 columns on the MoE token buffer
    w = workloads.fp8_col_experts()
    Rb, Cb = w.codes.shape[0], w.codes.shape[1] * 2
    Nb = Rb * Cb
    n = 2
    codes = [w.codes.to(dev) for _ in range(n)]
    e8 = [w.e8m0.to(dev) for _ in range(n)]
    off = torch.tensor(w.offsets, dtype=torch.int64, device=dev)
    outs = [mxq.mxq_fp4_row_to_fp8_col(codes[k], e8[k], off) for k in range(n)]
    outs = [(o[0].as_strided((Cb, Rb), (o[0].stride(0), 1)), o[1]) for o in outs]
    G = int(np.sum((np.diff(w.offsets) + 127) // 128))
    row("fp4_row_to_fp8_col", lambda k: mxq.mxq_fp4_row_to_fp8_col(codes[k], e8[k], off, out=outs[k]), n,
        Nb // 2 + Nb // 32 + Nb + 4 * Cb * G + 8 * len(w.offsets),
        f"{Rb}x{Cb} MXFP4 tokens of 256 experts (Dirichlet 0.5 split) -> E4M3 of the transpose, {G} groups")
    del codes, e8, outs
    torch.cuda.empty_cache()
    return rows, abl


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100, help="untimed steps (also bring the clocks up)")
    ap.add_argument("--kernel-reps", type=int, default=20, help="back-to-back launches per kernel for its duration")
    ap.add_argument("--single-reps", type=int, default=50,
                    help="individually timed launches per kernel (median, p10, p90)")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="rows of the oracle sample (0: skip)")
    ap.add_argument("--no-next", action="store_true", help="skip the rows beyond the step and the ablation")
    ap.add_argument("--configs", action="store_true",
                    help="also time every configuration at its own shape ([config] lines on stderr)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one MI355X: the quantisation kernels need no collectives and this "
              "build runs on a single GPU; --gpus must be 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from mxfp4_microscaling_quantization_amd import mxq, workloads

    mxq.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    R, C = 16384, 7168
    x_cpu = workloads.moe_activations(R, C, 2)
    x = x_cpu.to(dev)
    sets = 3
    kernels, (q8, s128) = build_step(x, dev, sets)
    step_bytes = sum(b for _, _, b in kernels)

    for w in range(args.warmup):
        for _, fn, _ in kernels:
            fn(w % sets)
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps, bracketed by events on torch's current stream.
    E = torch.cuda.Event
    start, stop = E(enable_timing=True), E(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for k in range(args.steps):
        for _, fn, _ in kernels:
            fn(k % sets)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(stop)
    ms_per_step = gpu_ms / args.steps
    value = step_bytes * args.steps / (gpu_ms / 1e3) / 1e9
    print(f"[bench] {args.steps} steps: {gpu_ms:.3f} ms on the stream ({wall * 1e3:.3f} ms wall), "
          f"{step_bytes / 1e6:.1f} MB per step", file=sys.stderr, flush=True)

    # Per-kernel average launch duration: `kernel_reps` back-to-back launches of one
    # kernel, rotating through the buffer sets, between two events on the stream the
    # kernels run on, so the events' own cost is spread over the launches. (Inside the
    # step a kernel also absorbs the write-back of its predecessor's output; the step
    # time above includes that.)
    per = {}
    for name, fn, b in kernels:
        fn(0)
        s0, s1 = E(enable_timing=True), E(enable_timing=True)
        s0.record()
        for r in range(args.kernel_reps):
            fn((r + 1) % sets)
        s1.record()
        torch.cuda.synchronize()
        us = s0.elapsed_time(s1) * 1e3 / args.kernel_reps
        gbs = b / (us * 1e-6) / 1e9
        per[name] = {"us": round(us, 3), "bytes": b, "GB_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        # the distribution of single launches: an event pair around each of
        # `single_reps` launches (recorded back to back, read after one synchronise)
        ev = [(E(enable_timing=True), E(enable_timing=True)) for _ in range(args.single_reps)]
        for r, (a, z) in enumerate(ev):
            a.record()
            fn((r + 1) % sets)
            z.record()
        torch.cuda.synchronize()
        one = np.array([a.elapsed_time(z) * 1e3 for a, z in ev])
        per[name].update({"us_p10": round(float(np.percentile(one, 10)), 3),
                          "us_median": round(float(np.median(one)), 3),
                          "us_p90": round(float(np.percentile(one, 90)), 3), "single_launches": len(one)})
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

    nxt, abl = (None, None)
    if not args.no_next:
        del kernels
        torch.cuda.empty_cache()
        nxt, abl = next_rows(dev, x)

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
        "next_rows": nxt,
        "ablation_fused_vs_unfused": abl,
    }
    if args.configs:
        torch.cuda.empty_cache()
        config_report(dev)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
