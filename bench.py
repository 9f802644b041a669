#!/usr/bin/env python3
"""Benchmark of the W8A8 quantized linear layer on one MI355X.

Prints ONE JSON line.  The headline (`value`) is the prefill FFN-up step
(q8_linear, X bf16 [2048, 4096] x W int8 [14336, 4096] -> bf16): per-token
INT8 activation quantization followed by the INT8 MFMA GEMM with its fused
dequantization epilogue, in int8 TOPS (2*M*N*K per step).  The weights are
quantized once before timing, as at model load.  The same line carries the
decode q_proj step (M = 16 and M = 1, N = K = 4096) in GB/s, the LLM.int8
decomposition and the FP8 rowwise step, each with the roofline of its
dominant kernel, and the CPU oracle timed on a bounded sample.

Timing: at least W untimed warm-up steps, continued until the leg has run
for 60 ms (the shader clock climbs over the first tens of milliseconds of
load; the JSON's `warmup` is the count actually run), then exactly K steps
between two stream synchronizations, timed with HIP events on the stream the
kernels run on.
Inside the timed region every launch of the dominant kernel is bracketed by
its own event pair; their mean is the kernel's average duration.  Decode
steps (a few microseconds each) are captured into a HIP graph over 32
distinct weight sets (537 MB, more than the 256 MB Infinity Cache) and
replayed, so host launch overhead and cache reuse do not enter the figure.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from w8a8_quantized_linear_channel_amd import inputs  # noqa: E402
from w8a8_quantized_linear_channel_amd import ops as q8  # noqa: E402

PEAK_INT8_TOPS = 5000.0       # dense int8 MFMA, MI355X
PEAK_FP8_TFLOPS = 5000.0      # dense fp8 MFMA, MI355X
PEAK_HBM_GBS = 8000.0         # HBM3E, MI355X
METRIC = "q8_linear int8 TOPS (prefill) + GB/s (decode) and % of MI355X roofline"


# HBM traffic of one launch of the prefill GEMM, from two rocprofv3 --pmc
# runs of `bench.py --only prefill --steps 3 --warmup 1 --warm-ms 0
# --no-cpu-baseline` (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each
# scaled by what the same counter reads for a plain 256 MiB device copy
# (`bench.py --only copy`): FETCH_SIZE reads 131087 KiB for 262144 KiB moved
# (x 2.0), WRITE_SIZE 262144 KiB (x 1.0).  Valid for the GEMM sources whose
# hash is recorded here; after any change to them the figure is withheld.
GEMM_TRAFFIC = {
    "sources_sha256": "c633bc8e3f88cf7144ffa8ccc3be81ee7c5aa6a62867f8bf8f75e448fba7d548",
    "fetch_kib": 90436.39, "fetch_scale": 262144.0 / 131085.40,
    "write_kib": 57359.77, "write_scale": 262144.0 / 262144.00,
}


def gemm_traffic_bytes():
    """Per-launch HBM bytes of the prefill GEMM, or None if its sources changed."""
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "w8a8_quantized_linear_channel_amd", "csrc")
    for f in ("gemm.hip", "q8_device.hpp", "q8_kernels.hpp"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    t = GEMM_TRAFFIC
    if h.hexdigest() != t["sources_sha256"]:
        return None
    return int((t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024)


def ev():
    return torch.cuda.Event(enable_timing=True)


# The shader clock climbs for the first few tens of milliseconds of sustained
# load (and again after the GPU idles): a quant+GEMM prefill step takes
# ~170 us at first and settles at ~120 us after ~200 steps.  Every leg is
# therefore warmed up until it has also run for WARM_MS, so that what is
# timed is the steady state a serving loop sees.
WARM_MS = 60.0


def set_warm_ms(ms):
    global WARM_MS
    WARM_MS = ms


def mark(pair, k):
    """Record event k of a step's pair around its dominant kernel (none in
    the regions timed without pairs)."""
    if pair is not None:
        pair[k].record()


def warm_up(step, warmup, min_ms=None):
    """Run `warmup` steps, then more (in groups of 8) until `min_ms` has
    passed on the GPU; return (steps run, ms)."""
    min_ms = WARM_MS if min_ms is None else min_ms
    t0, t1 = ev(), ev()
    t0.record()
    n = 0
    while True:
        for _ in range(max(1, warmup - n) if n < warmup else 8):
            step(n, None)
            n += 1
        t1.record()
        t1.synchronize()
        if n >= warmup and t0.elapsed_time(t1) >= min_ms:
            return n, t0.elapsed_time(t1)


def timed_steps(step, steps, warmup, kernel_pairs):
    """Warm up (at least `warmup` steps and WARM_MS), then time `steps` steps;
    return (ms per step, mean ms of the bracketed dominant kernel, (warm-up
    steps, warm-up ms)).  `step(i, pair)` must launch one step and, through
    `mark`, record pair[0]/pair[1] around the dominant kernel.

    The steps are timed twice, back to back.  The first region has no event
    inside: an event pair recorded between two kernels of a step adds ~6 us
    to it (measured on the prefill step: 125.6 us with a pair around the
    GEMM, 119.7 us without), so the step time comes from that region alone.
    The second region repeats the same steps with a pair around every
    dominant kernel, and gives its mean duration."""
    warm = warm_up(step, warmup)
    torch.cuda.synchronize()
    t0, t1 = ev(), ev()
    t0.record()
    for i in range(steps):
        step(i, None)
    t1.record()
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1)
    kern = None
    if kernel_pairs:
        for i in range(steps):
            step(i, kernel_pairs[i])
        torch.cuda.synchronize()
        kern = sum(a.elapsed_time(b) for a, b in kernel_pairs) / steps
    return total / steps, kern, warm


def graph_us(launch, n, replays):
    """Mean microseconds per call of `launch()`, captured n times in one HIP
    graph and replayed `replays` times after the usual warm-up."""
    launch()                        # first call outside the capture
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(n):
                launch()
    torch.cuda.synchronize()
    warm_up(lambda i, pair: g.replay(), 3)
    torch.cuda.synchronize()
    t0, t1 = ev(), ev()
    t0.record()
    for _ in range(replays):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / (n * replays)


# ------------------------------------------------------------------ prefill
def bench_prefill(dev, steps, warmup):
    wl = inputs.prefill_ffn_up()
    M, K = wl.x.shape
    N = wl.w.shape[0]
    x = wl.x.to(dev)
    wq, ws, wz = q8.q8_quantize_weight(wl.w.to(dev), "int8_asym")      # offline step
    xq = torch.empty(M, K, dtype=torch.int8, device=dev)
    xs = torch.empty(M, dtype=torch.float32, device=dev)
    xr = torch.empty(M, dtype=torch.int32, device=dev)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)

    def step(i, pair):
        q8.q8_quantize_act(x, "int8_sym", out=(xq, xs, xr))
        mark(pair, 0)
        q8.q8_gemm_int8(xq, xs, xr, wq, ws, wz, out_dtype=torch.bfloat16, out=y)
        mark(pair, 1)

    pairs = [(ev(), ev()) for _ in range(steps)]
    ms, gemm_ms, warm = timed_steps(step, steps, warmup, pairs)
    ops = 2.0 * M * N * K
    res = {
        "ms_per_step": ms,
        "tops": ops / (ms * 1e-3) / 1e12,
        "gemm_us": gemm_ms * 1e3,
        "gemm_tops": ops / (gemm_ms * 1e-3) / 1e12,
        "shape": (M, N, K),
        "warm": warm,
    }
    # act-quant kernel alone (HBM-bound): bytes = X bf16 in + codes out + 8 B/row.
    # Its launches are replayed from a HIP graph: launched one by one from
    # Python, the host's cost per call (~11 us) exceeds the kernel's, and
    # an event pair per launch costs a few microseconds more.
    q_us = graph_us(lambda: q8.q8_quantize_act(x, "int8_sym", out=(xq, xs, xr)), steps, 8)
    qbytes = M * K * 2 + M * K + 8 * M
    res["act_quant_us"] = q_us
    res["act_quant_gbs"] = qbytes / (q_us * 1e-6) / 1e9
    return res


# ------------------------------------------------------------------ decode
def bench_decode(dev, M, replays, copies=32, mode="w8a8", group=128):
    """Decode q_proj calls in graph replay over `copies` weight sets (beyond
    the caches).  mode: "w8a8" (q8_linear), "w8a16" (q8_linear_w8a16) or
    "grouped" (q8_linear_grouped with per-group weights)."""
    wl = inputs.decode_qproj(M=16)
    N, K = wl.w.shape
    x = wl.x[:M].contiguous().to(dev)
    weights = []
    for c in range(copies):
        w = (wl.w if c == 0 else inputs.decode_weight_copy(c, N, K)).to(dev)
        weights.append(q8.q8_quantize_weight_grouped(w, group) if mode == "grouped"
                       else q8.q8_quantize_weight(w, "int8_asym"))
    ys = [torch.empty(M, N, dtype=torch.bfloat16, device=dev) for _ in range(copies)]
    op = "grouped" if mode == "grouped" else "linear"
    wsp = torch.empty(max(1, q8.q8_workspace_bytes(op, M, N, K)), dtype=torch.uint8, device=dev)

    def one_pass():
        for c in range(copies):
            wq, wsc, wz = weights[c]
            if mode == "w8a16":
                q8.q8_linear_w8a16(x, wq, wsc, wz, out_dtype=torch.bfloat16, out=ys[c])
            elif mode == "grouped":
                q8.q8_linear_grouped(x, wq, wsc, wz, group, out_dtype=torch.bfloat16, out=ys[c], workspace=wsp)
            else:
                q8.q8_linear(x, wq, wsc, wz, out_dtype=torch.bfloat16, out=ys[c], workspace=wsp)

    one_pass()                      # warm up outside capture
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            one_pass()
    torch.cuda.synchronize()
    warm_up(lambda i, pair: g.replay(), 3)
    torch.cuda.synchronize()
    t0, t1 = ev(), ev()
    t0.record()
    for _ in range(replays):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    per_call_us = t0.elapsed_time(t1) * 1e3 / (replays * copies)
    params = 8 * N * (K // group) if mode == "grouped" else 8 * N
    nbytes = N * K + params + M * K * 2 + M * N * 2
    return {
        "M": M, "N": N, "K": K,
        "us_per_call": per_call_us,
        "gbs": nbytes / (per_call_us * 1e-6) / 1e9,
        "bytes_per_call": nbytes,
    }


# ------------------------------------------------------------------ LLM.int8
def bench_decomp(dev, steps, warmup):
    wl = inputs.llm_int8_outliers()
    M, K = wl.x.shape
    N = wl.w.shape[0]
    x = wl.x.to(dev)
    wq, ws, wz = q8.q8_quantize_weight(wl.w.to(dev), "int8_asym")
    y = torch.empty(M, N, dtype=torch.float16, device=dev)
    wsp = torch.empty(q8.q8_workspace_bytes("decomp", M, N, K), dtype=torch.uint8, device=dev)

    def step(i, pair):
        q8.q8_linear_int8_decomp(x, wq, ws, wz, 6.0, out=y, workspace=wsp)

    # no per-step events: at ~20 us a step, an event pair per step is a
    # visible share of it
    eager_ms, _, _ = timed_steps(step, steps, warmup, None)
    # The step time is taken from a HIP graph of 20 steps, as the decode legs
    # are: issued eagerly from Python, three launches of ~7 us each keep the
    # host about as busy as the GPU, and the eager figure varies by +-15 %
    # from run to run with the same library; it is reported beside it.
    ms = graph_us(lambda: q8.q8_linear_int8_decomp(x, wq, ws, wz, 6.0, out=y, workspace=wsp),
                  20, max(4, steps // 2)) * 1e-3
    ops = 2.0 * M * N * K
    nbytes = N * K + 8 * N + M * K * 2 + M * N * 2
    t_ideal = max(ops / (PEAK_INT8_TOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9))
    return {"M": M, "N": N, "K": K, "ms_per_step": ms, "eager_ms_per_step": eager_ms,
            "tops": ops / (ms * 1e-3) / 1e12,
            "roofline": {"bound": "ridge", "ideal_us": t_ideal * 1e6, "frac": t_ideal / (ms * 1e-3)}}


# ------------------------------------------------------------------ FP8
def bench_fp8(dev, steps, warmup):
    wl = inputs.fp8_rowwise()
    M, K = wl.x.shape
    N = wl.w.shape[0]
    x = wl.x.to(dev)
    wq, ws, _ = q8.q8_quantize_weight(wl.w.to(dev), "fp8_e4m3")
    xq = torch.empty(M, K, dtype=torch.uint8, device=dev)
    xs = torch.empty(M, dtype=torch.float32, device=dev)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)

    def step(i, pair):
        q8.q8_quantize_act(x, "fp8_e4m3", scale_ub=1200.0, out=(xq, xs, None))
        mark(pair, 0)
        q8.q8_gemm_fp8(xq, xs, wq, ws, out=y)
        mark(pair, 1)

    pairs = [(ev(), ev()) for _ in range(steps)]
    ms, gemm_ms, _ = timed_steps(step, steps, warmup, pairs)
    flops = 2.0 * M * N * K
    return {"M": M, "N": N, "K": K, "ms_per_step": ms, "tflops": flops / (ms * 1e-3) / 1e12,
            "gemm_us": gemm_ms * 1e3,
            "roofline": {"bound": "mfma", "achieved": flops / (gemm_ms * 1e-3) / 1e12,
                         "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                         "frac": flops / (gemm_ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS}}


# ------------------------------------------------------------------ FP8 experts on routed tokens
def bench_moe_fp8(dev, steps, warmup):
    """One FP8 expert projection over routed tokens (T = 4096 tokens, 8
    experts, N = K = 4096, Dirichlet-multinomial routing): per-token FP8
    quantization of all rows, then the grouped rowwise FP8 GEMM whose tiles
    follow the device-side expert offsets."""
    wl = inputs.moe_fp8()
    off = wl.extra["offsets"]
    E = off.numel() - 1
    T, K = wl.x.shape
    N = wl.w.shape[1]
    x = wl.x.to(dev)
    wq, ws, _ = q8.q8_quantize_weight(wl.w.reshape(E * N, K).to(dev), "fp8_e4m3")
    wq, ws = wq.view(E, N, K), ws.view(E, N)
    offd = off.to(dev)
    y = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
    wsp = torch.empty(q8.q8_workspace_bytes("fp8", T, N, K), dtype=torch.uint8, device=dev)

    def step(i, pair):
        q8.q8_linear_fp8_grouped(x, offd, wq, ws, scale_ub=1200.0, out=y, workspace=wsp)

    ms, _, _ = timed_steps(step, steps, warmup, None)
    flops = 2.0 * T * N * K
    return {"ms_per_step": ms, "tflops": flops / (ms * 1e-3) / 1e12, "tokens_per_expert": torch.diff(off).tolist(),
            "shape": (T, N, K, E)}


# ------------------------------------------------------------------ static scales, INT8 output
def bench_static(dev, steps, warmup):
    """Prefill FFN-up shape with a static activation scale and an INT8 output:
    q8_linear_static (static quantization kernel + int8 GEMM whose epilogue
    requantizes in float64)."""
    wl = inputs.prefill_ffn_up()
    M, K = wl.x.shape
    N = wl.w.shape[0]
    x = wl.x.to(dev)
    wq, ws, wz = q8.q8_quantize_weight(wl.w.to(dev), "int8_asym")
    yq = torch.empty(M, N, dtype=torch.int8, device=dev)
    wsp = torch.empty(q8.q8_workspace_bytes("static", M, N, K), dtype=torch.uint8, device=dev)
    x_scale, y_scale = 0.03, 0.05      # calibration stand-ins: |x| <= 3.8 on this data, |y| ~ 2

    def step(i, pair):
        q8.q8_linear_static(x, x_scale, wq, ws, wz, y_scale, out=yq, workspace=wsp)

    ms, _, _ = timed_steps(step, steps, warmup, None)
    ops = 2.0 * M * N * K
    return {"ms_per_step": ms, "tops": ops / (ms * 1e-3) / 1e12}


def bench_grouped(dev, steps, warmup, group=128):
    """Prefill FFN-up shape with per-group weights: q8_linear_grouped (row
    quantizer with group code sums + grouped GEMM)."""
    wl = inputs.prefill_ffn_up()
    M, K = wl.x.shape
    N = wl.w.shape[0]
    x = wl.x.to(dev)
    wq, ws, wz = q8.q8_quantize_weight_grouped(wl.w.to(dev), group)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    wsp = torch.empty(q8.q8_workspace_bytes("grouped", M, N, K), dtype=torch.uint8, device=dev)

    def step(i, pair):
        q8.q8_linear_grouped(x, wq, ws, wz, group, out=y, workspace=wsp)

    ms, _, _ = timed_steps(step, steps, warmup, None)
    ops = 2.0 * M * N * K
    return {"ms_per_step": ms, "tops": ops / (ms * 1e-3) / 1e12}


# ------------------------------------------------------------------ measured ceilings
def stream_read_ceiling(dev, steps):
    """HBM ceiling from the library's streaming-read kernel (include/q8_bench.h):
    the best of a few launch widths, (a) at 16.8 MB per launch -- the decode
    weight stream -- over 32 distinct buffers (537 MB, beyond the 256 MB
    Infinity Cache) replayed from a HIP graph as the decode calls are, and
    (b) one 512 MiB buffer per launch."""
    res = {}
    nb = 4096 * 4096 + 8 * 4096
    bufs = [torch.empty(nb, dtype=torch.uint8, device=dev).random_(0, 255) for _ in range(32)]
    best = None
    for wgs in (512, 1024, 2048):
        sink = torch.empty(wgs * 256, dtype=torch.int32, device=dev)
        us = graph_us(lambda: [q8.q8_bench_stream_read(b, wgs, sink) for b in bufs], 1, max(4, steps // 4))
        us /= len(bufs)
        if best is None or us < best[0]:
            best = (us, wgs)
    res["16.8MB_rotating_32_buffers"] = {"GB/s": round(nb / (best[0] * 1e-6) / 1e9, 1), "us": round(best[0], 3),
                                          "workgroups": best[1]}
    del bufs
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).random_(0, 255)
    best = None
    for wgs in (2048, 4096, 8192):
        sink = torch.empty(wgs * 256, dtype=torch.int32, device=dev)
        _, ms, _ = timed_steps(lambda i, pair: (mark(pair, 0), q8.q8_bench_stream_read(src, wgs, sink), mark(pair, 1)),
                               max(4, steps // 4), 2, [(ev(), ev()) for _ in range(max(4, steps // 4))])
        if best is None or ms < best[0]:
            best = (ms, wgs)
    res["512MiB"] = {"GB/s": round(n / (best[0] * 1e-3) / 1e9, 1), "us": round(best[0] * 1e3, 2), "workgroups": best[1]}
    del src
    return res


def bench_ceilings(dev, steps):
    """What this machine reaches with a streaming read and with the vendor
    GEMM library on the same shapes, beside the specification peaks: the
    streaming read for the HBM-bound rows, hipBLASLt (torch._int_mm with INT32
    output, torch._scaled_mm rowwise) for the GEMMs.  A ceiling is the best of three
    timed regions, each after the usual warm-up (the library's first region
    has been measured up to 20 % slower than its later ones)."""
    out = {}

    def t_ms(fn):
        best = None
        for _ in range(3):
            _, ms, _ = timed_steps(lambda i, pair: (mark(pair, 0), fn(), mark(pair, 1)), steps, 2,
                                   [(ev(), ev()) for _ in range(steps)])
            best = ms if best is None else min(best, ms)
        return best

    out["hbm_stream_read"] = stream_read_ceiling(dev, steps)
    g = torch.Generator(device="cpu").manual_seed(5)
    try:
        M, N, K = 2048, 14336, 4096
        a = (torch.randn(M, K, generator=g) * 30).round().clamp(-127, 127).to(torch.int8).to(dev)
        b = (torch.randn(N, K, generator=g) * 30).round().clamp(-127, 127).to(torch.int8).to(dev)
        ms = t_ms(lambda: torch._int_mm(a, b.t()))
        out["lib_int8_gemm_2048x14336x4096"] = {"us": round(ms * 1e3, 2), "TOPS": round(2 * M * N * K / (ms * 1e-3) / 1e12, 1),
                                                "output": "int32, no epilogue"}
    except Exception as e:  # the library call is context, not part of the path
        out["lib_int8_gemm_2048x14336x4096"] = f"unavailable: {str(e)[:80]}"
    try:
        M, N, K = 4096, 4096, 14336
        fa = torch.randn(M, K, generator=g).to(dev).to(torch.float8_e4m3fn)
        fb = torch.randn(N, K, generator=g).to(dev).to(torch.float8_e4m3fn)
        sa = torch.rand(M, 1, device=dev)
        sb = torch.rand(1, N, device=dev)
        ms = t_ms(lambda: torch._scaled_mm(fa, fb.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16))
        out["lib_fp8_rowwise_gemm_4096x4096x14336"] = {"us": round(ms * 1e3, 2),
                                                       "TFLOPS": round(2 * M * N * K / (ms * 1e-3) / 1e12, 1)}
    except Exception as e:
        out["lib_fp8_rowwise_gemm_4096x4096x14336"] = f"unavailable: {str(e)[:80]}"
    # register-only MFMA loops (include/q8_bench.h): the matrix-core rate with
    # no memory traffic, 512 workgroups (two waves per SIMD)
    sink = torch.empty(512 * 256, dtype=torch.int32, device=dev)
    for fmt, name, per in (("int8_sym", "mfma_loop_int8_TOPS", 65536), ("fp8_e4m3", "mfma_loop_fp8_TFLOPS", 131072)):
        iters = 4000
        ms = t_ms(lambda: q8.q8_bench_mfma_loop(fmt, iters, 512, sink))
        out[name] = round(512 * 4 * iters * 4 * per / (ms * 1e-3) / 1e12, 1)
    return out


# ------------------------------------------------------------------ CPU oracle
def _oracle_threads():
    """Threads the oracle's numpy uses (its BLAS pool does the matrix
    products; the rest of numpy is single-threaded)."""
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:   # threadpoolctl is optional: fall back to the host's count
        pass
    return os.cpu_count() or 1


def _time_rows(fn, rows_total, budget_s, min_rows=1):
    """Run fn(rows) on a small sample, then grow the sample (at most to
    rows_total) until a run takes at least half the budget; return (rows,
    seconds) of the last run."""
    rows = max(min_rows, min(rows_total, 8))
    while True:
        t = time.perf_counter()
        fn(rows)
        dt = time.perf_counter() - t
        if rows >= rows_total or dt >= 0.5 * budget_s:
            return rows, dt
        rows = int(min(rows_total, max(2 * rows, rows * 0.8 * budget_s / max(dt, 1e-3))))


def cpu_baselines(budget_s):
    """The oracle (oracle/q8_oracle.py, untuned numpy; its integer and FP8
    matrix products go to numpy's multi-threaded BLAS) on each workload's
    forward step, host inputs, weights quantized beforehand (untimed).  Each
    workload gets about budget_s seconds: the whole step if it fits, else the
    first R token rows against all the weights, scaled to the step's unit."""
    from oracle import q8_oracle as O
    cores = _oracle_threads()
    out = {}
    # prefill FFN-up (the headline workload)
    wl = inputs.prefill_ffn_up()
    wq, ws, wz = O.quantize_weight_int8_asym(wl.w)
    N, K = wl.w.shape
    rows, dt = _time_rows(lambda r: O.linear_int8(wl.x[:r], wq, ws, wz), wl.x.shape[0], budget_s)
    out["prefill"] = {"value": 2.0 * rows * N * K / dt / 1e12, "unit": "TOPS", "cores": cores, "kind": "oracle",
                      "seconds": dt, "sample": f"{rows} of {wl.x.shape[0]} token rows of the prefill FFN-up step "
                                              f"(activation quantization, exact integer GEMM, epilogue) against "
                                              f"all {N}x{K} weights"}
    del wq, ws, wz, wl
    # decode q_proj, M = 16: bytes as the GPU figure counts them
    wl = inputs.decode_qproj(M=16)
    wq, ws, wz = O.quantize_weight_int8_asym(wl.w)
    N, K = wl.w.shape
    reps, t = 0, time.perf_counter()
    while time.perf_counter() - t < min(budget_s, 3.0) or reps == 0:
        O.linear_int8(wl.x, wq, ws, wz)
        reps += 1
    dt = (time.perf_counter() - t) / reps
    nbytes = N * K + 8 * N + 16 * K * 2 + 16 * N * 2
    out["decode_M16"] = {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
                         "seconds": dt, "sample": f"the whole 16-token q_proj call, mean of {reps}"}
    del wq, ws, wz, wl
    # LLM.int8 decomposition
    wl = inputs.llm_int8_outliers()
    wq, ws, wz = O.quantize_weight_int8_asym(wl.w)
    N, K = wl.w.shape
    rows, dt = _time_rows(lambda r: O.linear_int8_decomp(wl.x[:r], wq, ws, wz, 6.0), wl.x.shape[0], budget_s, 64)
    out["llm_int8"] = {"value": 2.0 * rows * N * K / dt / 1e12, "unit": "TOPS", "cores": cores, "kind": "oracle",
                       "seconds": dt, "sample": f"{rows} of {wl.x.shape[0]} token rows (outlier columns found on "
                                                f"those rows) against all {N}x{K} weights"}
    del wq, ws, wz, wl
    # FP8 rowwise
    wl = inputs.fp8_rowwise()
    wq, ws = O.quantize_fp8_rowwise(wl.w)
    N, K = wl.w.shape
    rows, dt = _time_rows(lambda r: O.linear_fp8(wl.x[:r], wq, ws, 1200.0), wl.x.shape[0], budget_s)
    out["fp8"] = {"value": 2.0 * rows * N * K / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                  "seconds": dt, "sample": f"{rows} of {wl.x.shape[0]} token rows against all {N}x{K} weights"}
    del wq, ws, wl
    # tiny W8A8 linear
    wl = inputs.tiny_linear()
    wq, ws, wz = O.quantize_weight_int8_asym(wl.w)
    reps, t = 0, time.perf_counter()
    while time.perf_counter() - t < 0.5 or reps == 0:
        O.linear_int8(wl.x, wq, ws, wz)
        reps += 1
    dt = (time.perf_counter() - t) / reps
    M, K = wl.x.shape
    N = wl.w.shape[0]
    out["tiny"] = {"value": dt * 1e6, "unit": "us per call", "cores": cores, "kind": "oracle", "seconds": dt,
                   "sample": f"the whole {M}x{N}x{K} call, mean of {reps}"}
    return out


_T0 = time.time()


def progress(leg):
    """One line on stderr as each leg finishes; stdout keeps the single JSON line."""
    print(f"bench: {leg} done at {time.time() - _T0:.1f} s", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=400,
                    help="minimum warm-up steps per leg (each leg also warms up for %g ms)" % WARM_MS)
    ap.add_argument("--cpu-seconds", type=float, default=5.0,
                    help="host seconds per workload for the oracle's cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "decomp", "fp8", "moe", "static", "grouped", "copy"], default=None,
                    help="run one workload (for profiling); 'copy' runs a plain 256 MiB device copy, "
                         "the known-size kernel that scales the HBM byte counters")
    ap.add_argument("--warm-ms", type=float, default=WARM_MS,
                    help="minimum warm-up time per leg in ms (0 for counter runs)")
    args = ap.parse_args()
    set_warm_ms(args.warm_ms)
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    out = {"metric": METRIC}
    if args.only == "copy":
        n = 256 << 20
        src = torch.randint(0, 255, (n,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)
        return
    if args.only in (None, "prefill"):
        pf = bench_prefill(dev, args.steps, args.warmup)
        progress("prefill")
        M, N, K = pf["shape"]
        out.update({
            "value": round(pf["tops"], 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "warmup_steps_run": pf["warm"][0], "warmup_ms": round(pf["warm"][1], 1),
            "ms_per_step": round(pf["ms_per_step"], 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
            "data": "synthetic: seeded numpy PCG64, X ~ N(0,1) in bf16, W ~ N(0,0.02) quantized once",
            "config": {"workload": "prefill FFN-up q8_linear (dynamic per-token int8 X, per-channel "
                                   "asymmetric int8 W, INT32 accumulation, bf16 out)",
                       "M": M, "N": N, "K": K, "x_dtype": "bf16", "y_dtype": "bf16"},
            "roofline": {"bound": "mfma", "kernel": "k_gemm int8 256x256",
                         "achieved": round(pf["gemm_tops"], 1), "peak": PEAK_INT8_TOPS,
                         "unit": "TOP/s", "frac": round(pf["gemm_tops"] / PEAK_INT8_TOPS, 4),
                         "traffic": gemm_traffic_bytes(), "traffic_unit": "bytes per launch",
                         "algorithmic_bytes": M * K + N * K + 8 * N + 8 * M + 2 * M * N,
                         "kernel_us": round(pf["gemm_us"], 2)},
            "act_quant": {"us": round(pf["act_quant_us"], 2), "gbs": round(pf["act_quant_gbs"], 1),
                          "frac_hbm": round(pf["act_quant_gbs"] / PEAK_HBM_GBS, 4)},
        })
    if args.only in (None, "decode"):
        dec = {}
        for M in (16, 1):
            d = bench_decode(dev, M, replays=max(4, args.steps // 4))
            dec[f"M{M}"] = {"us_per_call": round(d["us_per_call"], 3), "GB/s": round(d["gbs"], 1),
                            "roofline": {"bound": "hbm", "achieved": round(d["gbs"], 1),
                                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                         "frac": round(d["gbs"] / PEAK_HBM_GBS, 4),
                                         "bytes_per_call": d["bytes_per_call"]}}
        out["decode"] = {"workload": "decode q_proj q8_linear, N = K = 4096, bf16, 32 rotating weight sets",
                         **dec}
        progress("decode")
        wo = {}
        for M in (16, 1):
            d = bench_decode(dev, M, replays=max(4, args.steps // 4), mode="w8a16")
            wo[f"M{M}"] = {"us_per_call": round(d["us_per_call"], 3), "GB/s": round(d["gbs"], 1),
                           "roofline": {"bound": "hbm", "achieved": round(d["gbs"], 1), "peak": PEAK_HBM_GBS,
                                        "unit": "GB/s", "frac": round(d["gbs"] / PEAK_HBM_GBS, 4),
                                        "bytes_per_call": d["bytes_per_call"]}}
        out["decode_w8a16"] = {"workload": "weight-only q8_linear_w8a16 decode q_proj, N = K = 4096, bf16 x, "
                                           "32 rotating weight sets", **wo}
        progress("decode_w8a16")
    if args.only in (None, "decomp"):
        d = bench_decomp(dev, args.steps, args.warmup)
        progress("llm_int8")
        out["llm_int8"] = {"workload": "LLM.int8 decomposition 512x4096x4096 fp16, 6 outlier columns",
                           "ms_per_step": round(d["ms_per_step"], 5), "timing": "HIP graph of 20 steps",
                           "eager_ms_per_step": round(d["eager_ms_per_step"], 5), "TOPS": round(d["tops"], 1),
                           "roofline": {k: round(v, 4) if isinstance(v, float) else v
                                        for k, v in d["roofline"].items()}}
    if args.only in (None, "fp8"):
        d = bench_fp8(dev, args.steps, args.warmup)
        progress("fp8")
        out["fp8"] = {"workload": "FP8 e4m3 rowwise 4096x4096x14336 bf16, scale_ub 1200",
                      "ms_per_step": round(d["ms_per_step"], 5), "TFLOPS": round(d["tflops"], 1),
                      "gemm_us": round(d["gemm_us"], 2),
                      "roofline": {k: round(v, 4) if isinstance(v, float) else v
                                   for k, v in d["roofline"].items()}}
    if args.only in (None, "moe"):
        d = bench_moe_fp8(dev, args.steps, args.warmup)
        progress("moe_fp8")
        T, N, K, E = d["shape"]
        out["moe_fp8"] = {"workload": f"FP8 expert projection, {T} routed tokens over {E} experts "
                                      f"{d['tokens_per_expert']}, N = K = {N}, bf16 out, ub 1200",
                          "ms_per_step": round(d["ms_per_step"], 5), "TFLOPS": round(d["tflops"], 1),
                          "frac_of_fp8_peak": round(d["tflops"] / PEAK_FP8_TFLOPS, 4)}
    if args.only in (None, "static"):
        d = bench_static(dev, args.steps, args.warmup)
        progress("static_int8_out")
        out["static_int8_out"] = {"workload": "prefill FFN-up 2048x14336x4096, static activation scale, INT8 output "
                                              "(q8_linear_static: static quantization + int8 GEMM, float64 requantize)",
                                  "ms_per_step": round(d["ms_per_step"], 5), "TOPS": round(d["tops"], 1),
                                  "frac_of_int8_peak": round(d["tops"] / PEAK_INT8_TOPS, 4)}
    if args.only is None:
        out["ceilings"] = bench_ceilings(dev, args.steps)
        progress("ceilings")
    if args.only in (None, "grouped"):
        d = bench_grouped(dev, args.steps, args.warmup)
        progress("grouped_prefill")
        out["grouped_prefill"] = {"workload": "prefill FFN-up 2048x14336x4096, per-group weights (group 128), "
                                              "q8_linear_grouped: row quantizer with group code sums + grouped GEMM",
                                  "ms_per_step": round(d["ms_per_step"], 5), "TOPS": round(d["tops"], 1),
                                  "frac_of_int8_peak": round(d["tops"] / PEAK_INT8_TOPS, 4)}
        gd = {}
        for M in (16, 1):
            d = bench_decode(dev, M, replays=max(4, args.steps // 4), mode="grouped")
            gd[f"M{M}"] = {"us_per_call": round(d["us_per_call"], 3), "GB/s": round(d["gbs"], 1),
                           "roofline": {"bound": "hbm", "achieved": round(d["gbs"], 1), "peak": PEAK_HBM_GBS,
                                        "unit": "GB/s", "frac": round(d["gbs"] / PEAK_HBM_GBS, 4),
                                        "bytes_per_call": d["bytes_per_call"]}}
        out["grouped_decode"] = {"workload": "q8_linear_grouped decode q_proj, N = K = 4096, group 128, bf16, "
                                             "32 rotating weight sets", **gd}
        progress("grouped_decode")
    if args.only in (None, "prefill") and not args.no_cpu_baseline:
        cb = cpu_baselines(args.cpu_seconds)
        progress("cpu_baseline")
        out["cpu_baseline"] = cb.pop("prefill")
        out["cpu_baseline_other_workloads"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
