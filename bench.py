"""Benchmark of the MXFP4 / NVFP4 quantise-and-convert hot path on one MI355X.

One step = one pass of the nine hot-path kernels, each over the synthetic workload
of the configuration it is quoted on (shapes of the pages' models: DeepSeek-V3-like
MoE with hidden 7168 and 256 experts; Llama-3.1-8B hidden 4096 / FFN 14336):
  moe_16384x7168       bf16 MoE activations       mxfp4_quantize, mxfp4_dequantize
  experts_65536x7168   FP8 token buffer           fp8_to_mxfp4, mxfp4_to_fp8
                       (256 experts, Dirichlet(0.5) split)
  grads_8192x14336     bf16 gradients             rht_mxfp4_rowcol (random-sign H16, row-
                       (N(0,1e-3) + Student-t(3)  and column-wise MXFP4 from one read)
                       noise)
  outliers_32768x4096  bf16 with outliers         nvfp4_amax, nvfp4_quantize_rne,
                                                  nvfp4_quantize_sr (Philox seed 7)
`value` = algorithmic bytes of the step (inputs read + outputs written, as the
method defines them) / the time of exactly `steps` steps. Each kernel is also timed
alone (`per_kernel`), beside a streaming kernel that moves the same bytes in the
same read/write mix (`stream_reference`: what that traffic reaches on this chip).
The small case small_1024x4096 (10.6 MB: launch-bound) is timed eagerly and from a HIP
graph. After the step the rows beyond it are timed at their own workloads, with the
fused-vs-unfused ablation of the FP8 <-> MXFP4 conversions; the CPU oracle is timed
on row samples of the same workloads (one core, then a pool of processes). Prints
one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
CUS, SIMDS_PER_CU, CLOCK_HZ = 256, 4, 2.4e9
# The published fp32 vector peak, 157.3 TFLOP/s = 256 CUs x 4 SIMDs x 32 lanes x 2
# flops x 2.4 GHz, means a SIMD retires a wave64 VALU instruction every 2 cycles: the
# chip issues at most CUS * SIMDS_PER_CU * CLOCK_HZ / 2 wave instructions per second.
VALU_WAVE_INST_PEAK = CUS * SIMDS_PER_CU * CLOCK_HZ / 2
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic.json")
VALU_FILE = os.path.join(PROFILES, "valu.json")
SOURCES = ("include/mxq.h", "mxfp4_microscaling_quantization_amd/csrc")


def source_digest() -> str:
    """SHA-256 over the library sources: PMC figures are reported only for the kernel
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


def committed_counters(path: str) -> dict:
    """Per-kernel PMC figures from a committed summary, if taken on these sources."""
    if not os.path.exists(path):
        return {}
    t = json.load(open(path))
    return t.get("kernels", {}) if t.get("source_sha256") == source_digest() else {}


# ---------------------------------------------------------------------------
# workloads

def load_workloads():
    """The seeded inputs of every configuration (CPU tensors), in a fixed order."""
    from mxfp4_microscaling_quantization_amd import workloads as W

    t0 = time.perf_counter()
    w = {"small_1024x4096": W.mxfp4_rowwise_small(), "moe_16384x7168": W.mxfp4_rowwise_moe(), "experts_65536x7168": W.fp8_moe_experts(),
         "grads_8192x14336": W.rht_gradients(), "outliers_32768x4096": W.nvfp4_activations()}
    print(f"[bench] workloads generated in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    return w


def mx_bytes(n):  # bf16 in, MXFP4 codes + E8M0 out (or the reverse)
    return 2 * n + n // 2 + n // 32


def fp8_bytes(n):  # E4M3 + 1x128 fp32 scales <-> MXFP4
    return n + 4 * (n // 128) + n // 2 + n // 32


def nv_bytes(n):  # bf16 in, NVFP4 codes + E4M3 block scales + fp32 tensor scale out
    return 2 * n + n // 2 + n // 16 + 4


class Kernel:
    """One timed kernel: fn(k) launches it on buffer set k; `mix` names its streaming
    reference (read bytes per unit, write bytes per unit, load/store flags)."""

    def __init__(self, name, cfg, shape, fn, nbytes, elements, mix, read_bytes):
        self.name, self.cfg, self.shape, self.fn = name, cfg, shape, fn
        self.bytes, self.elements, self.mix, self.read_bytes = nbytes, elements, mix, read_bytes


def build_step(wl, dev, sets: int):
    """The nine kernels of one step over `sets` independent buffer sets: within a set
    every kernel reads its own copy of its input, and launches rotate through the sets,
    so no launch finds its input in the 256 MB MALL or the L2 (a set is about 3.4 GB)."""
    import torch

    from mxfp4_microscaling_quantization_amd import mxq

    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16

    def e(*shape, dtype=u8):
        return torch.empty(shape, dtype=dtype, device=dev)

    x2, x4, x5 = wl["moe_16384x7168"].x.to(dev), wl["grads_8192x14336"].x.to(dev), wl["outliers_32768x4096"].x.to(dev)
    q8, s128 = wl["experts_65536x7168"].q8.to(dev), wl["experts_65536x7168"].s128.to(dev)
    R2, C2 = x2.shape
    R3, C3 = q8.shape
    R4, C4 = x4.shape
    R5, C5 = x5.shape
    seed4, seed5 = wl["grads_8192x14336"].rht_seed, wl["outliers_32768x4096"].sr_seed
    S = []
    for k in range(sets):
        st = {"x2q": x2 if k == 0 else x2.clone(), "q8": q8 if k == 0 else q8.clone(), "s128": s128.clone(),
              "x4": x4 if k == 0 else x4.clone(), "x5a": x5 if k == 0 else x5.clone(), "x5n": x5.clone(),
              "x5s": x5.clone()}
        st["deq_in"] = mxq.mxq_quantize(st["x2q"], "mxfp4", "row")
        st["f8_in"] = mxq.mxq_fp8_to_mxfp4(st["q8"], st["s128"])
        st["qz"] = mxq.Quantized(e(R2, C2 // 2), e(R2, C2 // 32), None, None, None)
        st["yb"] = e(R2, C2, dtype=bf)
        st["c8"] = (e(R3, C3 // 2), e(R3, C3 // 32))
        st["f8"] = (e(R3, C3), e(R3, C3 // 128, dtype=f32))
        st["rq"] = mxq.Quantized(e(R4, C4 // 2), e(R4, C4 // 32), e(C4, R4 // 2), e(C4, R4 // 32), None)
        st["amax"] = e(1, dtype=f32)
        st["nq"] = mxq.Quantized(e(R5, C5 // 2), e(R5, C5 // 16), None, None, e(1, dtype=f32))
        st["sq"] = mxq.Quantized(e(R5, C5 // 2), e(R5, C5 // 16), None, None, e(1, dtype=f32))
        S.append(st)
    torch.cuda.synchronize()
    n2, n3, n4, n5 = R2 * C2, R3 * C3, R4 * C4, R5 * C5
    sh2, sh3, sh4, sh5 = f"{R2}x{C2}", f"{R3}x{C3}", f"{R4}x{C4}", f"{R5}x{C5}"
    ks = [
        Kernel("mxfp4_quantize", "moe_16384x7168", sh2,
               lambda k: mxq.mxq_quantize(S[k]["x2q"], "mxfp4", "row", out=S[k]["qz"]),
               mx_bytes(n2), n2, (16, 4, 1), 2 * n2),
        Kernel("mxfp4_dequantize", "moe_16384x7168", sh2,
               lambda k: mxq.mxq_dequantize(S[k]["deq_in"].codes_row, S[k]["deq_in"].scales_row, "mxfp4",
                                            out=S[k]["yb"]),
               mx_bytes(n2), n2, (4, 16, 3), n2 // 2),
        Kernel("fp8_to_mxfp4", "experts_65536x7168", sh3,
               lambda k: mxq.mxq_fp8_to_mxfp4(S[k]["q8"], S[k]["s128"], out=S[k]["c8"]),
               fp8_bytes(n3), n3, (16, 8, 1), n3),
        Kernel("mxfp4_to_fp8", "experts_65536x7168", sh3,
               lambda k: mxq.mxq_mxfp4_to_fp8(S[k]["f8_in"][0], S[k]["f8_in"][1], out=S[k]["f8"]),
               fp8_bytes(n3), n3, (8, 16, 3), n3 // 2),
        Kernel("rht_mxfp4_rowcol", "grads_8192x14336", sh4,
               lambda k: mxq.mxq_rht_quantize(S[k]["x4"], seed4, "mxfp4", "both", out=S[k]["rq"]),
               2 * n4 + 2 * (n4 // 2 + n4 // 32), n4, ("strip",), 2 * n4),
        Kernel("nvfp4_amax", "outliers_32768x4096", sh5,
               lambda k: mxq.mxq_amax(S[k]["x5a"], out=S[k]["amax"]), 2 * n5 + 4, n5, (16, 0, 1), 2 * n5),
        Kernel("nvfp4_quantize_rne", "outliers_32768x4096", sh5,
               lambda k: mxq.mxq_quantize(S[k]["x5n"], "nvfp4", "row", amax=S[k]["amax"], out=S[k]["nq"]),
               nv_bytes(n5), n5, (16, 4, 1), 2 * n5),
        Kernel("nvfp4_quantize_sr", "outliers_32768x4096", sh5,
               lambda k: mxq.mxq_quantize(S[k]["x5s"], "nvfp4", "row", "sr", sr_seed=seed5, amax=S[k]["amax"],
                                          out=S[k]["sq"]),
               nv_bytes(n5), n5, (16, 4, 1), 2 * n5),
    ]
    for k in range(sets):  # the amax every NVFP4 quantisation of the set reads
        mxq.mxq_amax(S[k]["x5a"], out=S[k]["amax"])
    torch.cuda.synchronize()
    return ks


# ---------------------------------------------------------------------------
# timing helpers

_busy = None
_counters_mode = False  # set by --counters: every dispatch is serialised by the profiler


def keep_busy(dev, seconds: float = 0.25) -> None:
    """Keeps the GPU busy for `seconds` with a compute-only kernel (no memory traffic),
    so the measurement that follows does not start on a clock that dropped while the
    host prepared its buffers (a few hundred ms idle lowers it; kernels bound by the
    vector ALU then run up to 25 % slower)."""
    import torch

    global _busy
    if _counters_mode:
        return
    L = stream_lib()
    if _busy is None:
        _busy = torch.empty(2048, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            L.mxq_valu_probe(_busy.data_ptr(), 2048, 256, 0, st)
        torch.cuda.synchronize()


def avg_launch_us(fn, sets: int, reps: int) -> float:
    """Average duration of `reps` back-to-back launches rotating over the buffer sets,
    between two events on the stream the kernels run on (torch's current stream)."""
    import torch

    E = torch.cuda.Event
    fn(0)
    a, b = E(enable_timing=True), E(enable_timing=True)
    a.record()
    for r in range(reps):
        fn((r + 1) % sets)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / reps


def single_launch_us(fn, sets: int, reps: int):
    """p10 / median / p90 of `reps` individually timed launches (an event pair around
    each, read after one synchronisation)."""
    import numpy as np
    import torch

    E = torch.cuda.Event
    ev = [(E(enable_timing=True), E(enable_timing=True)) for _ in range(reps)]
    for r, (a, z) in enumerate(ev):
        a.record()
        fn((r + 1) % sets)
        z.record()
    torch.cuda.synchronize()
    one = np.array([a.elapsed_time(z) * 1e3 for a, z in ev])
    return {"us_p10": round(float(np.percentile(one, 10)), 3), "us_median": round(float(np.median(one)), 3),
            "us_p90": round(float(np.percentile(one, 90)), 3), "single_launches": int(len(one))}


def figures(us: float, nbytes: int, elements: int) -> dict:
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us": round(us, 3), "bytes": int(nbytes), "GB_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "elements_per_s": round(elements / (us * 1e-6), 1)}


# ---------------------------------------------------------------------------
# streaming references (libmxq_stream.so)

_stream_lib = None


def stream_lib():
    global _stream_lib
    if _stream_lib is None:
        p = os.path.join(ROOT, "mxfp4_microscaling_quantization_amd", "libmxq_stream.so")
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is missing: build it with `python -m mxfp4_microscaling_quantization_amd.build`")
        L = ctypes.CDLL(p)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        L.mxq_stream_mix.argtypes = [vp, vp, i64, i32, i32, i32, vp]
        L.mxq_stream_strip_pattern.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp]
        L.mxq_stream_2d_pattern.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp]
        L.mxq_valu_probe.argtypes = [vp, i32, i32, i32, vp]
        for n in ("mxq_stream_mix", "mxq_stream_strip_pattern", "mxq_stream_2d_pattern", "mxq_valu_probe"):
            getattr(L, n).restype = i32
        _stream_lib = L
    return _stream_lib


def stream_mix_reference(dev, read_bytes: int, rd: int, wr: int, flags: int, reps: int, sets: int = 3) -> dict:
    """A plain streaming kernel reading `read_bytes` (rd bytes per lane unit) and
    writing wr/rd as many, over rotating buffer sets: the fastest of 1, 2 and 4 lane
    units per thread (write-heavy mixes stream faster with fewer)."""
    best = None
    for u, code in ((4, 0), (2, 2), (1, 1)):
        r = _stream_mix_once(dev, read_bytes, rd, wr, flags | (code << 2), reps, sets)
        r["lane_units_per_thread"] = u
        if best is None or r["us"] < best["us"]:
            best = r
    return best


def _stream_mix_once(dev, read_bytes: int, rd: int, wr: int, flags: int, reps: int, sets: int) -> dict:
    import torch

    L = stream_lib()
    units = read_bytes // rd
    src = [torch.empty(units * rd, dtype=torch.uint8, device=dev).fill_(k + 1) for k in range(sets)]
    dst = [torch.empty(max(units * wr, (units // 1024 + 1) * 4), dtype=torch.uint8, device=dev) for _ in range(sets)]
    st = torch.cuda.current_stream().cuda_stream

    def fn(k):
        rc = L.mxq_stream_mix(src[k].data_ptr(), dst[k].data_ptr(), units, rd, wr, flags, st)
        if rc:
            raise RuntimeError(f"mxq_stream_mix({rd}, {wr}) returned {rc}")

    for k in range(sets):
        fn(k)
    keep_busy(dev)
    us = avg_launch_us(fn, sets, reps)
    nbytes = units * (rd + wr)
    out = figures(us, nbytes, units)
    out.pop("elements_per_s")
    out.update({"read_per_unit": rd, "write_per_unit": wr, "nontemporal_loads": bool(flags & 1),
                "nontemporal_stores": bool(flags & 2)})
    del src, dst
    torch.cuda.empty_cache()
    return out


def pattern_reference(dev, kind: str, rows: int, cols: int, reps: int, sets: int = 3) -> dict:
    """A fused row + column kernel's access pattern, moving bytes only: kind "strip" (the
    bf16 MXFP4 row + column strip kernel) or "2d" (16x16 NVFP4, W and W^T)."""
    import torch

    L = stream_lib()
    bs = 32 if kind == "strip" else 16
    e = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)  # noqa: E731
    xs = [torch.full((rows, cols), k + 1, dtype=torch.bfloat16, device=dev) for k in range(sets)]
    outs = [(e(rows, cols // 2), e(rows, cols // bs), e(cols, rows // 2), e(cols, rows // bs)) for _ in range(sets)]
    st = torch.cuda.current_stream().cuda_stream
    call = L.mxq_stream_strip_pattern if kind == "strip" else L.mxq_stream_2d_pattern

    def fn(k):
        o = outs[k]
        rc = call(xs[k].data_ptr(), rows, cols, o[0].data_ptr(), o[1].data_ptr(), o[2].data_ptr(), o[3].data_ptr(), st)
        if rc:
            raise RuntimeError(f"{kind} pattern reference returned {rc}")

    for k in range(sets):
        fn(k)
    keep_busy(dev)
    us = avg_launch_us(fn, sets, reps)
    n = rows * cols
    out = figures(us, 2 * n + 2 * (n // 2 + n // bs), n)
    out.pop("elements_per_s")
    out.update({"pattern_kind": kind, "shape": f"{rows}x{cols}"})
    del xs, outs
    torch.cuda.empty_cache()
    return out


def valu_probe(dev, reps: int = 5) -> dict:
    """Wave instructions per second the chip retires for the integer instructions of
    the stochastic-rounding path (v_add_u32, v_bitop3_b32, v_mad_u64_u32)."""
    import torch

    L = stream_lib()
    blocks, iters = CUS * SIMDS_PER_CU * 8 // 4, 2048  # 8 waves per SIMD
    out = torch.empty(blocks, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    res = {}
    keep_busy(dev)
    for kind, name in ((0, "v_add_u32"), (1, "v_bitop3_b32"), (2, "v_mad_u64_u32")):
        fn = lambda k: L.mxq_valu_probe(out.data_ptr(), blocks, iters, kind, st)  # noqa: E731
        fn(0)
        us = avg_launch_us(fn, 1, reps)
        winst = blocks * 4 * 8 * iters  # 4 waves per workgroup, 8 instructions per iteration
        res[name] = {"us": round(us, 3), "wave_instructions": winst,
                     "wave_inst_per_s": round(winst / (us * 1e-6) / 1e9, 1),
                     "frac_of_issue_peak": round(winst / (us * 1e-6) / VALU_WAVE_INST_PEAK, 4)}
    res["issue_peak_wave_inst_per_s"] = round(VALU_WAVE_INST_PEAK / 1e9, 1)
    res["unit"] = "G wave instructions/s"
    return res


# ---------------------------------------------------------------------------
# the small case, the rows beyond the step, the ablation

def small_case_report(wl, dev, reps: int, graph: bool = True) -> list:
    """1024 x 4096 (10.6 MB): 64 rotating buffer sets, eager launches and the same
    launches replayed from a captured HIP graph (device time without the host's
    per-call cost)."""
    import torch

    from mxfp4_microscaling_quantization_amd import mxq

    n = 64
    xs = [wl["small_1024x4096"].x.to(dev) for _ in range(n)]
    R, C = xs[0].shape
    N = R * C
    qs = [mxq.mxq_quantize(x, "mxfp4", "row") for x in xs]
    ys = [torch.empty_like(x) for x in xs]
    qfn = lambda k: mxq.mxq_quantize(xs[k], "mxfp4", "row", out=qs[k])  # noqa: E731
    dfn = lambda k: mxq.mxq_dequantize(qs[k].codes_row, qs[k].scales_row, "mxfp4", out=ys[k])  # noqa: E731

    def graph_us(fn):
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
        E = torch.cuda.Event
        a, b = E(enable_timing=True), E(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    out = []
    for name, fn in (("mxfp4_quantize", qfn), ("mxfp4_dequantize", dfn)):
        for k in range(n):
            fn(k)
        keep_busy(dev)
        r = {"config": "small_1024x4096", "kernel": name, "shape": f"{R}x{C}", "launch": "eager"}
        r.update(figures(avg_launch_us(fn, n, reps), mx_bytes(N), N))
        out.append(r)
        if graph:
            r = {"config": "small_1024x4096", "kernel": name, "shape": f"{R}x{C}", "launch": "hip_graph"}
            r.update(figures(graph_us(fn), mx_bytes(N), N))
            out.append(r)
    del xs, qs, ys
    return out


def extra_rows(wl, dev, reps: int, traffic: dict, refs: bool = True) -> tuple[dict, dict]:
    """The rows beyond the step, each at its own workload with rotating input copies:
    NVFP4 amax + quantise as one call (the amax computed by the call), 16x16-scaled
    NVFP4 of a 14336 x 4096 FFN weight (both outputs), RHT + NVFP4 column-wise and
    MXFP4 stochastic rounding of the 8192x14336 gradients, the MXFP4-rows -> FP8-columns
    conversion of the 65536 x 7168 token buffer of 256 experts; and the fused-vs-
    unfused ablation of the FP8 <-> MXFP4 conversions on the 65536x7168 token buffer."""
    import numpy as np
    import torch

    from mxfp4_microscaling_quantization_amd import mxq, workloads

    rows = {}

    def row(name, cfg, shape, fn, n, nbytes, elements, note):
        for k in range(n):
            fn(k)
        keep_busy(dev)
        us = avg_launch_us(fn, n, reps)
        r = {"config": cfg, "shape": shape, "workload": note}
        r.update(figures(us, nbytes, elements))
        t = traffic.get(name, {}).get("hbm_bytes")
        r["hbm_traffic_bytes"] = t
        r["traffic_ratio"] = round(t / nbytes, 4) if t else None
        rows[name] = r
        print(f"[next] {name:28s} {us:9.2f} us  {r['GB_s']:8.1f} GB/s  {100 * r['frac_hbm_peak']:5.1f}%",
              file=sys.stderr, flush=True)
        return us

    n = 3
    # NVFP4 end to end: one call that computes the amax first (two passes over x)
    x5 = [wl["outliers_32768x4096"].x.to(dev) for _ in range(n)]
    R5, C5 = x5[0].shape
    N5 = R5 * C5
    o5 = [mxq.mxq_quantize(v, "nvfp4", "row") for v in x5]
    row("nvfp4_amax_quantize_rne", "outliers_32768x4096", f"{R5}x{C5}",
        lambda k: mxq.mxq_quantize(x5[k], "nvfp4", "row", out=o5[k]), n, nv_bytes(N5), N5,
        "amax pass + quantise pass in one call (NULL amax); bytes = the quantiser's in+out, "
        "so the two-pass ceiling is 2.5625 / 4.5625 of the HBM peak")
    a5 = [mxq.mxq_amax(v) for v in x5]
    row("nvfp4_quantize_sr16", "outliers_32768x4096", f"{R5}x{C5}",
        lambda k: mxq.mxq_quantize(x5[k], "nvfp4", "row", "sr16", sr_seed=wl["outliers_32768x4096"].sr_seed, amax=a5[k],
                                   out=o5[k]), n, nv_bytes(N5), N5,
        "NVFP4 stochastic rounding, opt-in 16-bit-halves random stream (one Philox call per 8 elements)")
    del x5, o5, a5
    # 16x16 NVFP4 of an FFN weight
    wt = workloads.outlier_normal(14336, 4096, 5)
    ws = [wt.to(dev) for _ in range(n)]
    am = [mxq.mxq_amax(v) for v in ws]
    Rw, Cw = wt.shape
    Nw = Rw * Cw
    q2 = [mxq.mxq_quantize(v, "nvfp4_2d", "both", amax=a) for v, a in zip(ws, am)]
    row("nvfp4_2d_rowcol", "ffn_weight", f"{Rw}x{Cw}",
        lambda k: mxq.mxq_quantize(ws[k], "nvfp4_2d", "both", amax=am[k], out=q2[k]), n,
        2 * Nw + 2 * (Nw // 2 + Nw // 16) + 4, Nw, "14336x4096 FFN weight (outlier law, seed 5), 16x16 block "
        "scales, W and W^T codes from one read")
    del ws, am, q2
    if refs:  # what the kernel's access pattern reaches when it moves bytes only
        ref = pattern_reference(dev, "2d", Rw, Cw, reps)
        rows["nvfp4_2d_rowcol"]["stream_ref_GB_s"] = ref["GB_s"]
        rows["nvfp4_2d_rowcol"]["frac_of_stream_ref"] = round(rows["nvfp4_2d_rowcol"]["GB_s"] / ref["GB_s"], 4)
        rows["nvfp4_2d_rowcol"]["stream_ref_pattern"] = "16x16 NVFP4 tile pattern, bytes only"
        print(f"[ref]   nvfp4_2d_rowcol {ref['GB_s']:8.1f} GB/s (16x16 NVFP4 tile pattern); kernel at "
              f"{100 * rows['nvfp4_2d_rowcol']['frac_of_stream_ref']:.1f}%", file=sys.stderr, flush=True)
    # gradient recipes on the grads_8192x14336 tensor
    x4 = [wl["grads_8192x14336"].x.to(dev) for _ in range(n)]
    R4, C4 = x4[0].shape
    N4 = R4 * C4
    mask = mxq.mxq_rht_signs(wl["grads_8192x14336"].rht_seed)
    ra = [mxq.mxq_rht_amax(v, mask, "col") for v in x4]
    rq = [mxq.mxq_rht_quantize(v, wl["grads_8192x14336"].rht_seed, "nvfp4", "col", amax=a) for v, a in zip(x4, ra)]
    row("rht_nvfp4_col", "grads_8192x14336", f"{R4}x{C4}",
        lambda k: mxq.mxq_rht_quantize(x4[k], wl["grads_8192x14336"].rht_seed, "nvfp4", "col", amax=ra[k], out=rq[k]), n,
        nv_bytes(N4), N4, "H16 along rows, column-wise NVFP4 (the wgrad recipe)")
    row("rht_amax_col", "grads_8192x14336", f"{R4}x{C4}", lambda k: mxq.mxq_rht_amax(x4[k], mask, "col", out=ra[k]), n,
        2 * N4 + 4, N4, "amax of the column-wise transform")
    del rq
    sq = [mxq.mxq_quantize(v, "mxfp4", "row") for v in x4]
    row("mxfp4_quantize_sr", "grads_8192x14336", f"{R4}x{C4}",
        lambda k: mxq.mxq_quantize(x4[k], "mxfp4", "row", "sr", sr_seed=7, out=sq[k]), n, mx_bytes(N4), N4,
        "row-wise MXFP4, Philox stochastic rounding (gradients)")
    row("mxfp4_quantize_sr16", "grads_8192x14336", f"{R4}x{C4}",
        lambda k: mxq.mxq_quantize(x4[k], "mxfp4", "row", "sr16", sr_seed=7, out=sq[k]), n, mx_bytes(N4), N4,
        "row-wise MXFP4, stochastic rounding with the opt-in 16-bit-halves stream")
    rcol = [(torch.empty((C4, R4 // 2), dtype=torch.uint8, device=dev),
             torch.empty((C4, R4 // 32), dtype=torch.uint8, device=dev)) for _ in range(n)]
    row("mxfp4_rowcol_no_rht", "grads_8192x14336", f"{R4}x{C4}",
        lambda k: mxq.mxq_quantize(x4[k], "mxfp4", "both", out=mxq.Quantized(sq[k].codes_row, sq[k].scales_row,
                                                                              rcol[k][0], rcol[k][1], None)),
        n, 2 * N4 + 2 * (N4 // 2 + N4 // 32), N4, "the fused row + column kernel without the transform")
    del x4, ra, sq, rcol
    torch.cuda.empty_cache()

    # ---- fused vs unfused on the experts_65536x7168 buffer (the pages' kernel-level claim)
    abl = {}
    n = 2
    q8 = [wl["experts_65536x7168"].q8.to(dev) for _ in range(n)]
    s128 = [wl["experts_65536x7168"].s128.to(dev) for _ in range(n)]
    R3, C3 = q8[0].shape
    N3 = R3 * C3
    f_out = [mxq.mxq_fp8_to_mxfp4(q8[k], s128[k]) for k in range(n)]
    yb = [torch.empty((R3, C3), dtype=torch.bfloat16, device=dev) for _ in range(n)]
    cz = [(torch.empty((R3, C3 // 2), dtype=torch.uint8, device=dev),
           torch.empty((R3, C3 // 32), dtype=torch.uint8, device=dev)) for _ in range(n)]

    def fp8_unfused(k):
        v = q8[k].view(torch.float8_e4m3fn).to(torch.bfloat16).view(R3, C3 // 128, 128)
        torch.mul(v, s128[k].to(torch.bfloat16)[..., None], out=yb[k].view(R3, C3 // 128, 128))
        return mxq.mxq_quantize(yb[k], "mxfp4", "row", out=mxq.Quantized(cz[k][0], cz[k][1], None, None, None))

    fb = fp8_bytes(N3)
    ideal = (N3 + 4 * (N3 // 128) + 2 * N3 + 2 * N3 + N3 // 2 + N3 // 32) / fb
    t_f = row("fp8_to_mxfp4 (fused)", "experts_65536x7168", f"{R3}x{C3}",
              lambda k: mxq.mxq_fp8_to_mxfp4(q8[k], s128[k], out=f_out[k]), n, fb, N3, "E4M3 + 1x128 scales")
    t_u = row("fp8_to_mxfp4 (unfused)", "experts_65536x7168", f"{R3}x{C3}", fp8_unfused, n, fb, N3,
              "torch E4M3->bf16 cast and scaling, then mxq_quantize")
    u = fp8_unfused(0)
    torch.cuda.synchronize()
    same = bool(torch.equal(u.codes_row, f_out[0][0]) and torch.equal(u.scales_row, f_out[0][1]))
    abl["fp8_to_mxfp4"] = {"fused_us": round(t_f, 3), "unfused_us": round(t_u, 3), "speedup": round(t_u / t_f, 3),
                           "same_bits": same, "unfused_to_fused_bytes": round(ideal, 3), "shape": f"{R3}x{C3}"}
    b_out = [mxq.mxq_mxfp4_to_fp8(*f_out[k]) for k in range(n)]
    q8o = [torch.empty((R3, C3), dtype=torch.uint8, device=dev) for _ in range(n)]

    def mx_unfused(k):
        mxq.mxq_dequantize(f_out[k][0], f_out[k][1], "mxfp4", out=yb[k])
        smax = f_out[k][1].view(R3, C3 // 128, 4).amax(-1).to(torch.int32)
        sc = torch.ldexp(torch.ones((), device=dev), (smax - 127).float())
        q = torch.div(yb[k].view(R3, C3 // 128, 128).float(), sc[..., None]).to(torch.float8_e4m3fn)
        q8o[k].copy_(q.view(torch.uint8).view(R3, C3))
        return q8o[k], sc

    t_f = row("mxfp4_to_fp8 (fused)", "experts_65536x7168", f"{R3}x{C3}", lambda k: mxq.mxq_mxfp4_to_fp8(*f_out[k], out=b_out[k]),
              n, fb, N3, "MXFP4 -> E4M3 + 1x128 scales")
    t_u = row("mxfp4_to_fp8 (unfused)", "experts_65536x7168", f"{R3}x{C3}", mx_unfused, n, fb, N3,
              "mxq_dequantize to bf16, then torch scaling and E4M3 cast")
    uq, us_ = mx_unfused(0)
    torch.cuda.synchronize()
    same = bool(torch.equal(uq, b_out[0][0]) and torch.equal(us_.float(), b_out[0][1]))
    abl["mxfp4_to_fp8"] = {"fused_us": round(t_f, 3), "unfused_us": round(t_u, 3), "speedup": round(t_u / t_f, 3),
                           "same_bits": same, "unfused_to_fused_bytes": round(ideal, 3), "shape": f"{R3}x{C3}"}
    del q8, s128, f_out, yb, cz, b_out, q8o
    torch.cuda.empty_cache()

    # ---- MXFP4 rows -> FP8 columns on the MoE token buffer
    w = workloads.fp8_col_experts()
    Rb, Cb = w.codes.shape[0], w.codes.shape[1] * 2
    Nb = Rb * Cb
    codes = [w.codes.to(dev) for _ in range(n)]
    e8 = [w.e8m0.to(dev) for _ in range(n)]
    off = torch.tensor(w.offsets, dtype=torch.int64, device=dev)
    outs = [mxq.mxq_fp4_row_to_fp8_col(codes[k], e8[k], off) for k in range(n)]
    outs = [(o[0].as_strided((Cb, Rb), (o[0].stride(0), 1)), o[1]) for o in outs]
    G = int(np.sum((np.diff(w.offsets) + 127) // 128))
    row("fp4_row_to_fp8_col", "experts_65536x7168", f"{Rb}x{Cb}",
        lambda k: mxq.mxq_fp4_row_to_fp8_col(codes[k], e8[k], off, out=outs[k]), n,
        Nb // 2 + Nb // 32 + Nb + 4 * Cb * G + 8 * len(w.offsets), Nb,
        f"MXFP4 tokens of 256 experts (the split of the 65536x7168 buffer) -> E4M3 of the transpose, {G} groups of 128 tokens")
    # the same buffer split into 256 experts of 256 tokens: every group starts on a
    # 128-byte output line (how much of the time the ragged split's unaligned group
    # runs cost)
    off_al = torch.arange(0, Rb + 1, Rb // 256, dtype=torch.int64, device=dev)
    G_al = Rb // 128
    row("fp4_row_to_fp8_col_aligned_experts", "experts_65536x7168", f"{Rb}x{Cb}",
        lambda k: mxq.mxq_fp4_row_to_fp8_col(codes[k], e8[k], off_al, out=outs[k]), n,
        Nb // 2 + Nb // 32 + Nb + 4 * Cb * G_al + 8 * 257, Nb,
        "the same buffer as 256 experts of 256 tokens (every group line-aligned): the cost of unaligned experts")
    del codes, e8, outs
    torch.cuda.empty_cache()
    return rows, abl


# ---------------------------------------------------------------------------
# CPU oracle baseline

_CPU = {}


def _oracle_step(part: int) -> int:
    """The oracle counterparts of the nine step kernels on rows [part*n, (part+1)*n) of
    each configuration's workload (row counts in _CPU['rows']); returns the bytes the
    step's byte accounting gives those rows."""
    import numpy as np

    from oracle import fp8 as ofp8
    from oracle import mx as omx
    from oracle import nvfp4 as onv
    from oracle import philox as oph
    from oracle import rht as orht

    def window(a, r):  # part's rows (windows wrap when the pool covers more than the tensor)
        start = (part * r) % max(1, a.shape[0] - r + 1)
        start -= start % 32
        return start, a[start:start + r]

    nb = 0
    r2, r3, r4, r5 = _CPU["rows"]
    _, x2 = window(_CPU["x2"], r2)
    c, e = omx.mxfp4_quantize_rowwise(x2)
    omx.mxfp4_dequantize(c, e, "bf16")
    nb += 2 * mx_bytes(x2.size)
    i3, q8 = window(_CPU["q8"], r3)
    s = _CPU["s3"][i3:i3 + r3]
    c8, e8 = ofp8.fp8_to_mxfp4(q8, s)
    ofp8.mxfp4_to_fp8(c8, e8)
    nb += 2 * fp8_bytes(q8.size)
    _, x4 = window(_CPU["x4"], r4)
    mask = _CPU["mask"]
    omx.mxfp4_quantize_rowwise(orht.rht_rowwise(x4, mask))
    omx.mxfp4_quantize_rowwise(orht.rht_rowwise(np.ascontiguousarray(x4.T), mask))
    nb += 2 * x4.size + 2 * (x4.size // 2 + x4.size // 32)
    i5, x5 = window(_CPU["x5"], r5)
    A = onv.tensor_amax(x5)
    onv.nvfp4_quantize_rowwise(x5, amax=A)
    R5, C5 = x5.shape
    onv.nvfp4_quantize_rowwise(x5, amax=A, r16=oph.tensor_r16(R5, C5, seed=7, offset=i5 * C5))
    nb += 2 * x5.size + 4 + 2 * nv_bytes(x5.size)
    return nb


def cpu_baseline(wl, rows: tuple, pool_size: int) -> dict | None:
    """The oracle as it stands on row samples of the step's workloads: one process,
    then `pool_size` processes each on its own rows (forked before the GPU is used)."""
    import multiprocessing as mp

    import numpy as np

    from oracle import rht as orht

    r2, r3, r4, r5 = rows
    _CPU["rows"] = rows
    f64 = lambda t: t.float().double().numpy()  # noqa: E731
    _CPU["x2"] = f64(wl["moe_16384x7168"].x)
    _CPU["q8"] = wl["experts_65536x7168"].q8.numpy()
    _CPU["s3"] = wl["experts_65536x7168"].s128.numpy().view(np.uint32)
    _CPU["x4"] = f64(wl["grads_8192x14336"].x)
    _CPU["x5"] = f64(wl["outliers_32768x4096"].x)
    _CPU["mask"] = orht.sign_mask_from_seed(wl["grads_8192x14336"].rht_seed)
    t0 = time.perf_counter()
    nb1 = _oracle_step(0)
    t1 = time.perf_counter() - t0
    single = nb1 / t1 / 1e9
    print(f"[bench] oracle, one process: {single:.4f} GB/s in {t1:.1f} s", file=sys.stderr, flush=True)
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    res = {"value": round(single, 4), "unit": "GB/s", "cores": 1, "kind": "oracle", "cpu_model": model,
           "sample": f"the nine kernels' oracle counterparts on rows of each workload ({r2} of moe_16384x7168, {r3} of experts_65536x7168, "
                     f"{r4} of grads_8192x14336, {r5} of outliers_32768x4096), {t1:.1f} s, one process (numpy elementwise is single-threaded)"}
    if pool_size > 1:
        ctx = mp.get_context("fork")
        with ctx.Pool(pool_size) as pool:
            t0 = time.perf_counter()
            nbs = pool.map(_oracle_step, range(pool_size))
            tp = time.perf_counter() - t0
        pooled = sum(nbs) / tp / 1e9
        print(f"[bench] oracle, {pool_size} processes: {pooled:.4f} GB/s in {tp:.1f} s", file=sys.stderr, flush=True)
        res["single_process"] = {"value": res["value"], "cores": 1, "seconds": round(t1, 2)}
        res.update({"value": round(pooled, 4), "cores": pool_size,
                    "sample": f"the nine kernels' oracle counterparts, {pool_size} processes (multiprocessing "
                              f"pool, one per core of the affinity mask, at most 16), each on its own window of "
                              f"rows of each workload ({r2} of moe_16384x7168, {r3} of experts_65536x7168, {r4} of grads_8192x14336, {r5} of outliers_32768x4096; "
                              f"windows wrap where the pool covers more than a tensor), {tp:.1f} s"})
    _CPU.clear()
    return res


# ---------------------------------------------------------------------------

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100, help="untimed steps (also bring the clocks up)")
    ap.add_argument("--kernel-reps", type=int, default=20, help="back-to-back launches per kernel for its duration")
    ap.add_argument("--single-reps", type=int, default=50,
                    help="individually timed launches per kernel (median, p10, p90)")
    ap.add_argument("--cpu-scale", type=float, default=1.0,
                    help="size of the oracle's row samples (1.0: about 10 s per process; 0: skip)")
    ap.add_argument("--cpu-procs", type=int, default=0, help="oracle pool size (0: the affinity mask, at most 16)")
    ap.add_argument("--no-next", action="store_true", help="skip the rows beyond the step and the ablation")
    ap.add_argument("--no-refs", action="store_true", help="skip the streaming references and the VALU probe")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph timing of configuration 1")
    ap.add_argument("--counters", action="store_true",
                    help="for rocprofv3 --pmc passes: no clock-holding busy loops, no graph timing, and of the "
                         "references only the 1 GiB copy (which scales FETCH_SIZE / WRITE_SIZE) and the VALU probe")
    args = ap.parse_args()
    if args.counters:
        global _counters_mode
        _counters_mode = True
        args.no_graph = True
    if args.gpus != 1:
        print("bench.py measures one MI355X: the quantisation kernels need no collectives and this "
              "build runs on a single GPU; --gpus must be 1", file=sys.stderr)
        return 2

    wl = load_workloads()
    cpu = None
    if args.cpu_scale > 0:  # before the GPU is touched: the pool forks this process
        procs = args.cpu_procs or min(16, len(os.sched_getaffinity(0)))
        s = args.cpu_scale
        rows = (max(32, int(4608 * s) // 32 * 32), max(32, int(4608 * s) // 32 * 32),
                max(32, int(2304 * s) // 32 * 32), max(32, int(8064 * s) // 32 * 32))
        cpu = cpu_baseline(wl, rows, procs)

    import torch

    from mxfp4_microscaling_quantization_amd import mxq

    mxq.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sets = 3
    kernels = build_step(wl, dev, sets)
    step_bytes = sum(k.bytes for k in kernels)

    for w in range(args.warmup):
        for k in kernels:
            k.fn(w % sets)
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps, bracketed by events on torch's current
    # stream (the stream every kernel is launched on).
    E = torch.cuda.Event
    start, stop = E(enable_timing=True), E(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for s in range(args.steps):
        for k in kernels:
            k.fn(s % sets)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(stop)
    ms_per_step = gpu_ms / args.steps
    value = step_bytes * args.steps / (gpu_ms / 1e3) / 1e9
    print(f"[bench] {args.steps} steps: {gpu_ms:.3f} ms on the stream ({wall * 1e3:.3f} ms wall), "
          f"{step_bytes / 1e6:.1f} MB per step", file=sys.stderr, flush=True)

    traffic = committed_counters(TRAFFIC_FILE)
    valu_counts = committed_counters(VALU_FILE)
    per, elements = {}, {}
    for k in kernels:
        key = f"{k.cfg}.{k.name}"
        us = avg_launch_us(k.fn, sets, args.kernel_reps)
        r = {"config": k.cfg, "shape": k.shape}
        r.update(figures(us, k.bytes, k.elements))
        r.update(single_launch_us(k.fn, sets, args.single_reps))
        t = traffic.get(key, {}).get("hbm_bytes")
        r["hbm_traffic_bytes"] = t
        r["traffic_ratio"] = round(t / k.bytes, 4) if t else None
        per[key] = r
        elements[key] = k.elements
        print(f"[bench] {key:26s} {us:9.2f} us  {r['GB_s']:8.1f} GB/s  {100 * r['frac_hbm_peak']:5.1f}% of 8 TB/s",
              file=sys.stderr, flush=True)

    refs, valu_ref = None, None
    if not args.no_refs:
        refs = {}
        for k in ([] if args.counters else kernels):
            key = f"{k.cfg}.{k.name}"
            if k.mix[0] == "strip":
                R, C = (int(v) for v in k.shape.split("x"))
                ref = pattern_reference(dev, "strip", R, C, args.kernel_reps)
                ref["pattern"] = "fused row + column strip pattern: 256-column strips, whole 128-byte column-code lines"
            else:
                rd, wr, fl = k.mix
                ref = stream_mix_reference(dev, k.read_bytes, rd, wr, fl, args.kernel_reps)
                ref["pattern"] = f"read {rd} B + write {wr} B per lane unit"
            refs[key] = ref
            per[key]["stream_ref_GB_s"] = ref["GB_s"]
            per[key]["frac_of_stream_ref"] = round(per[key]["GB_s"] / ref["GB_s"], 4)
            print(f"[ref]   {key:26s} {ref['GB_s']:8.1f} GB/s ({ref['pattern']}); kernel at "
                  f"{100 * per[key]['frac_of_stream_ref']:.1f}%", file=sys.stderr, flush=True)
        refs["copy_1GiB"] = stream_mix_reference(dev, 1 << 30, 16, 16, 3, args.kernel_reps)
        refs["copy_1GiB"]["pattern"] = "copy, 16 B per lane unit"
        valu_ref = valu_probe(dev)
        print(f"[ref]   VALU probe {json.dumps(valu_ref)}", file=sys.stderr, flush=True)

    # the roofline of the kernel that takes the longest (all of these are HBM-bound by
    # their arithmetic intensity; stochastic rounding also carries an issue analysis)
    dom = max(per, key=lambda k: per[k]["us"])
    d = per[dom]
    roof = {"kernel": dom, "bound": "hbm", "achieved": d["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": d["frac_hbm_peak"], "traffic": d["hbm_traffic_bytes"], "bytes_per_launch": d["bytes"],
            "avg_launch_us": d["us"], "workload": d["config"],
            "stream_ref_GB_s": d.get("stream_ref_GB_s")}

    # VALU issue analysis of the stochastic-rounding kernels from committed SQ counters
    valu = {}
    for key in per:
        c = valu_counts.get(key)
        if not c:
            continue
        winst = c["valu_wave_insts"]
        rate = winst / (per[key]["us"] * 1e-6)
        valu[key] = {"valu_wave_insts_per_launch": winst,
                     "valu_insts_per_element": round(winst * 64 / elements[key], 3),
                     "wave_inst_per_s": round(rate / 1e9, 1), "frac_of_issue_peak": round(rate / VALU_WAVE_INST_PEAK, 4)}
        if valu_ref:  # against what independent v_add_u32 chains reach on this chip
            valu[key]["frac_of_probe_rate"] = round(rate / (valu_ref["v_add_u32"]["wave_inst_per_s"] * 1e9), 4)
    if valu_ref:
        valu["probe"] = valu_ref

    small = small_case_report(wl, dev, args.kernel_reps, graph=not args.no_graph)
    for r in small:
        print(f"[small_1024x4096]  {r['kernel']:18s} {r['launch']:9s} {r['us']:8.2f} us  {100 * r['frac_hbm_peak']:5.1f}%",
              file=sys.stderr, flush=True)

    nxt, abl = (None, None)
    if not args.no_next:
        del kernels
        torch.cuda.empty_cache()
        nxt, abl = extra_rows(wl, dev, args.kernel_reps, traffic, refs=not (args.no_refs or args.counters))

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
        "config": {"workload": "mxfp4_nvfp4_hot_path_per_workload: the nine quantise/convert kernels per step, "
                               "each on its own workload (moe_16384x7168: bf16 MoE activations; experts_65536x7168: "
                               "FP8 tokens of 256 experts; grads_8192x14336: bf16 gradients; outliers_32768x4096: "
                               "bf16 with outliers)",
                   "bytes_per_step": step_bytes, "elements_per_step": sum(elements.values())},
        "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "per_kernel": per,
        "small_case": small,
        "roofline": roof,
        "valu": valu or None,
        "stream_reference": refs,
        "cpu_baseline": cpu,
        "next_rows": nxt,
        "ablation_fused_vs_unfused": abl,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
