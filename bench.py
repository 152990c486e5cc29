#!/usr/bin/env python
"""Benchmark of the HiLS attention hot path on one MI355X.

Headline (``value``): prefill tokens/s of the 8K workload (B=1, H=16, d=64,
L=8192, C=64, k=8, chunk-mean landmarks with four needle chunks).  One step is
one ``hils_sparse_attn_fwd`` call: scoring + top-k, routing, chunk attention,
own-chunk attention and fusion, with inputs resident in HBM.  The same JSON
line carries the 128K prefill, the 512K-context decode (cold-cache protocol:
R independent caches, one per emulated layer) and the 8K training step
(forward + backward), each with its per-kernel times.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip decode_512k,...]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s @8K & 128K; decode µs/token + HBM GB/s @512K ctx"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- measured HBM traffic
# FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the dominant kernel of each workload, from
# rocprofv3 --pmc runs of this script (the commands and tables are in profiles/).  FETCH_SIZE
# reads half the bytes a plain 1 GiB copy moves and WRITE_SIZE all of them, so the traffic is
# 2*FETCH + WRITE.  Each entry records a digest of the kernel's sources when the counters were
# taken; once the sources differ the entry no longer describes the kernel and traffic is null.
COUNTER_SCALE = {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
KERNEL_SOURCES = {
    "chunk_attn_fwd": "attn_fwd.hip", "own_combine": "attn_fwd.hip", "topk_select": "scores_topk.hip",
    "decode_scan": "decode.hip", "decode_attend": "decode.hip", "chunk_bwd": "attn_bwd.hip",
    "dq_reduce": "attn_bwd.hip", "klm_bwd": "attn_bwd.hip", "route_scatter": "route.hip",
}
MEASURED_TRAFFIC = {
    # workload: {kernel: (FETCH_SIZE KiB, WRITE_SIZE KiB, source digest)}
    "prefill_8k": {"chunk_attn_fwd": (28601.2, 130610.5, "a3092f13320f3339"), "topk_select": (8439.4, 13824.4, "586a724baeaea988"), "own_combine": (92234.5, 16384.0, "a3092f13320f3339")},
    "prefill_128k": {"chunk_attn_fwd": (8157821.3, 17023151.8, "a3092f13320f3339"), "topk_select": (533198.6, 835609.2, "586a724baeaea988"), "own_combine": (10197152.7, 1048576.0, "a3092f13320f3339")},
    "train_8k": {"chunk_bwd": (235663.0, 898528.4, "f4de254081963b9c"), "chunk_attn_fwd": (105704.4, 522515.0, "a3092f13320f3339"), "dq_reduce": (326648.0, 149726.5, "f4de254081963b9c")},
    "decode_512k": {"decode_scan": (8264.2, 68.0, "8aa435acddc0f2e9"), "decode_attend": (2434.7, 34.1, "8aa435acddc0f2e9")},
}


def kernel_source_digest(kernel):
    import hashlib

    h = hashlib.sha256()
    src = os.path.join(ROOT, "long_context_landmark_amd", "csrc")
    for f in (KERNEL_SOURCES[kernel], "hils_device.h"):
        with open(os.path.join(src, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch of the kernel from the recorded counters, or None."""
    rec = MEASURED_TRAFFIC.get(workload, {}).get(kernel)
    if rec is None or kernel_source_digest(kernel) != rec[2]:
        return None
    return round((rec[0] * COUNTER_SCALE["FETCH_SIZE"] + rec[1] * COUNTER_SCALE["WRITE_SIZE"]) * 1024)


# ----------------------------------------------------------------------------- algorithmic work
# Per kernel: (bound, algorithmic FLOPs, algorithmic bytes, design bytes).  "Algorithmic" is the method's own
# work: the landmark dot products (2d per causal (query, chunk) score), the attention inside each kept chunk
# (4 C d per (query, kept chunk) pair; causal for the own chunk) and reading Q, K, V, landmarks and writing O
# once.  "Design bytes" is this implementation's traffic model of the kernel (per-pair query gathers and
# partial-output round trips of the chunk-major schedule), reported beside the measured counter bytes; it is
# never used as achieved work.  Contractions are priced against bf16 MFMA, the rest against HBM.


def prefill_work(B, H, L, d, k, C=64):
    """Algorithmic FLOPs and bytes of one prefill forward, total and per kernel."""
    BH, N = B * H, L // C
    pairs = BH * C * sum(min(k, c) for c in range(N))
    f_topk = BH * 2 * d * (C * N * (N - 1) // 2 + L)
    f_chunk = pairs * 4 * C * d
    f_own = BH * N * 4 * d * (C * (C + 1) // 2)
    io = BH * (4 * L * d * 2 + N * d * 2)
    k1 = k + 1
    return {
        "pairs": pairs,
        "flops": f_topk + f_chunk + f_own,
        "bytes": io,
        "kernels": {
            # name: (bound, algorithmic flops, algorithmic bytes, design bytes)
            "topk_select": ("mfma", f_topk, BH * (L * d * 2 + N * d * 2), BH * (L * d * 2 + N * d * 2 + L * k1 * 12)),
            "chunk_attn_fwd": ("mfma", f_chunk, BH * L * d * 2 * 2,
                               pairs * (2 * d + 2 * d + 8) + BH * N * C * d * 4),
            "own_combine": ("hbm", f_own, BH * L * 4 * d * 2, BH * L * (3 * d * 2 + d * 2 + k1 * 8) + pairs * 2 * d),
            "route_count": ("hbm", 0, BH * L * k * 4, BH * L * k * 4),
            "route_scan": ("hbm", 0, BH * 2 * N * 4 * max(1, L // 1024), BH * 2 * N * 4 * max(1, L // 1024)),
            "route_scatter": ("hbm", 0, BH * L * k * 8, BH * L * k * 8),
            # landmark-free chunks only
            "chunk_mean": ("hbm", 0, BH * (L * d * 2 + N * d * 2), BH * (L * d * 2 + N * d * 2)),
            "lf_own": ("hbm", BH * L * 2 * d, BH * L * 2 * d * 2, BH * L * (2 * d * 2 + k1 * 12)),
            # two landmarks per chunk only: causal (query, chunk, landmark) dot products on MFMA in the
            # selection kernel, which reads the queries and both landmark rows of every chunk
            "topk_select_ml": ("mfma", BH * C * (N * (N + 1) // 2) * 2 * 2 * d, BH * (L * d * 2 + N * 2 * d * 2),
                               BH * (L * d * 2 + N * 2 * d * 2 + L * k1 * 12)),
        },
    }


def decode_work(B, H, d, n, k, C=64):
    BH = B * H
    c = n // C
    m = min(k, c)
    own = n - c * C + 1
    b_scan = BH * c * d * 2
    b_attn = BH * (m * C + own) * d * 2 * 2
    return {
        "bytes": b_scan + b_attn + BH * d * 2 * 5,
        "flops": BH * (2 * d * (c + 1) + 4 * d * (m * C + own)),
        "kernels": {"decode_scan": ("hbm", BH * 2 * d * c, b_scan, b_scan),
                    "decode_attend": ("hbm", BH * 4 * d * (m * C + own), b_attn, b_attn + BH * 64 * 16 * 8)},
    }


def train_work(B, H, L, d, k, C=64):
    fw = prefill_work(B, H, L, d, k, C)
    BH, N = B * H, L // C
    pairs_all = fw["pairs"] + BH * L
    f_bwd = (fw["pairs"] * 10 * C * d) + BH * N * 10 * d * (C * (C + 1) // 2)
    b_bwd = BH * L * (4 * d * 2 + 3 * d * 4) + BH * N * d * (2 + 4)  # Q, K, V, dO read; dQ, dK, dV, dKlm written
    kern = dict(fw["kernels"])
    kern["chunk_bwd"] = ("mfma", f_bwd, BH * L * (4 * d * 2 + 2 * d * 4),
                         pairs_all * (2 * d * 2 + 4 * d + 12) + BH * N * C * d * (2 * 2 + 4 * 2))
    kern["dq_reduce"] = ("hbm", 0, BH * L * d * 4, pairs_all * (4 * d + 2 * d + 12) + BH * L * d * 4)
    kern["klm_bwd"] = ("hbm", 0, BH * N * d * 4, pairs_all * (2 * d + 8) + BH * N * d * 4)
    # landmark-free chunks only: q and k read, dQ and dK read and written, per row
    kern["lf_bwd"] = ("hbm", 0, BH * L * 2 * d * 2, BH * L * (2 * d * 2 + 4 + 4 * d * 4) + BH * N * d * 4)
    # two landmarks per chunk only: per pair q read, the chunk's two landmark rows read and dKlm written
    kern["ml_klm_bwd"] = ("hbm", 0, BH * N * 2 * d * 4, pairs_all * (2 * d + 4) + BH * N * 2 * d * (2 + 4))
    return {"flops": fw["flops"] + f_bwd, "bytes": fw["bytes"] + b_bwd, "kernels": kern}


def roofline(kernels_ms, work, launches_per_step, workload=None, by_bytes=False):
    """Roofline of the kernel with the largest time per step (by_bytes: the largest algorithmic bytes, for
    the decode step, whose kernels last a few microseconds each, so that the HIP-event brackets, which add
    a launch's dispatch latency to each, would decide the choice).

    achieved = the kernel's algorithmic FLOPs (contractions, against bf16 MFMA) or bytes (against HBM) per
    launch over its average launch time from HIP events on the launching stream; traffic = HBM bytes per
    launch from the recorded FETCH_SIZE / WRITE_SIZE counters (null once the kernel's sources changed), and
    hbm_measured their rate over the same launch time."""
    if not kernels_ms:
        return None
    if by_bytes:
        name = max(kernels_ms, key=lambda n: work["kernels"].get(n, ("hbm", 0, 0, 0))[2])
    else:
        name = max(kernels_ms, key=lambda n: kernels_ms[n][0])
    total_ms, calls = kernels_ms[name]
    per_launch_ms = total_ms / max(1, calls)
    bound, flops, nbytes, design = work["kernels"].get(name, ("hbm", 0, 0, 0))
    per = max(1, launches_per_step.get(name, 1))
    if bound == "mfma":
        achieved = flops / per / (per_launch_ms * 1e-3) / 1e12
        peak, unit = PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved = nbytes / per / (per_launch_ms * 1e-3) / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
    traffic = measured_traffic(workload, name)
    out = {"kernel": name, "bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
           "frac": round(achieved / peak, 5), "traffic": traffic, "avg_launch_us": round(per_launch_ms * 1e3, 3),
           "design_bytes": int(design / per)}
    if traffic:
        gbs = traffic / (per_launch_ms * 1e-3) / 1e9
        out["hbm_measured"] = {"GB/s": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)}
    return out


def step_fractions(work, ms):
    """Whole-step algorithmic rates against both roofs."""
    tf = work["flops"] / (ms * 1e-3) / 1e12
    gbs = work["bytes"] / (ms * 1e-3) / 1e9
    return {"tflops": round(tf, 2), "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4), "hbm_gbs": round(gbs, 1),
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}


# ----------------------------------------------------------------------------- timing


def timed(fn, steps, warmup):
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(st)
    for _ in range(steps):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def timed_graph(fn, steps, warmup):
    """Capture one call of fn in a HIP graph and time ``steps`` replays (no host launch overhead)."""
    import torch

    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(st)
    for _ in range(steps):
        g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall, g


def host_ahead():
    """Queue a spin kernel of about 20 ms (5e7 shader clocks) so that the host enqueues the profiled
    launches while the GPU is busy.  The library then times each launch with events that its own dispatch
    records; when the host lags (a few hundred eager decode launches from Python take several ms), the
    GPU idles between kernels and those intervals grow by the idle time's dispatch and clock ramp."""
    import torch

    torch.cuda._sleep(int(5e7))


def kernel_times(hils, fn, steps):
    import torch

    torch.cuda.synchronize()
    hils.profile_enable(True)
    host_ahead()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    res = hils.profile_read()
    hils.profile_enable(False)
    return res


# ----------------------------------------------------------------------------- workloads


def bench_prefill(hils, synth, name, steps, warmup, rq=False, lf=False, ml=False):
    """rq: separate retrieval queries score the landmarks (low-rank query calibration).
    lf: landmark-free chunks, the landmarks formed inside the step as the chunks' key means."""
    import torch

    w = synth.WORKLOADS[name]
    x = synth.torch_prefill_inputs(w, with_qret=rq)
    klm_out = torch.empty_like(x["Klm"]) if lf else None
    # several landmarks per chunk: the keys of each chunk's first and last token
    klm_ml = torch.stack([x["K"][:, :, ::w.C], x["K"][:, :, w.C - 1::w.C]], dim=3).contiguous() if ml else None
    ws = torch.empty(hils.workspace_size(hils.OP_FWD_ML if ml else hils.OP_FWD, w.B, w.H, w.L, w.d, w.C, w.k), dtype=torch.uint8,
                     device="cuda:0")
    O = torch.empty_like(x["Q"])

    def step():
        if ml:
            hils.sparse_attn_fwd_ml(x["Q"], x["K"], x["V"], klm_ml, w.k, ws=ws, out=O, Q_ret=x.get("Q_ret"))
        elif lf:
            hils.sparse_attn_fwd_lf(x["Q"], x["K"], x["V"], w.k, ws=ws, out=O, Q_ret=x.get("Q_ret"), K_lm=klm_out)
        else:
            hils.sparse_attn_fwd(x["Q"], x["K"], x["V"], x["Klm"], w.k, ws=ws, out=O, Q_ret=x.get("Q_ret"))

    ms_eager, _ = timed(step, steps, warmup)
    ms, wall, graph = timed_graph(step, steps, warmup)
    del graph
    kt = kernel_times(hils, step, max(1, min(steps, 10)))
    work = prefill_work(w.B, w.H, w.L, w.d, w.k, w.C)
    nsteps = max(1, min(steps, 10))
    per_kernel = {n: round(t / c * 1e3, 3) for n, (t, c) in kt.items()}
    rl = roofline(kt, work, {n: c // nsteps for n, (t, c) in kt.items()}, None if rq or lf or ml else name)
    res = {
        "tokens_per_s": w.B * w.L / (ms * 1e-3),
        "ms_per_step": ms,
        "ms_per_step_eager": ms_eager,
        "timing": "HIP graph of one step, replayed",
        "wall_s": wall,
        "step_roofline": step_fractions(work, ms),
        "algorithmic_gflop": work["flops"] / 1e9,
        "algorithmic_mb": work["bytes"] / 1e6,
        "pairs": work["pairs"],
        "kernel_us": per_kernel,
        "roofline": rl,
        "config": {"workload": name, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "C": w.C, "k": w.k,
                   **({"retrieval_query": True} if rq else {}), **({"landmark_free": True} if lf else {}),
                   **({"landmarks_per_chunk": 2} if ml else {})},
    }
    del x, ws, O
    torch.cuda.empty_cache()
    return res


def bench_train(hils, synth, name, steps, warmup, rq=False, lf=False, ml=False):
    import torch

    w = synth.WORKLOADS[name]
    x = synth.torch_prefill_inputs(w, with_dO=True, with_qret=rq)
    wsf = torch.empty(hils.workspace_size(hils.OP_FWD, w.B, w.H, w.L, w.d, w.C, w.k), dtype=torch.uint8,
                      device="cuda:0")
    wsb = torch.empty(hils.workspace_size(hils.OP_BWD, w.B, w.H, w.L, w.d, w.C, w.k), dtype=torch.uint8,
                      device="cuda:0")

    # outputs of forward and backward are allocated once so the step can be replayed from a graph
    B, H, L, d, k1 = w.B, w.H, w.L, w.d, w.k + 1
    f32 = dict(dtype=torch.float32, device="cuda:0")
    O = torch.empty_like(x["Q"])
    idx = torch.empty((B, H, L, k1), dtype=torch.int32, device="cuda:0")
    sel, wt, lse = (torch.empty((B, H, L, k1), **f32) for _ in range(3))
    grads = [torch.empty((B, H, L, d), **f32) for _ in range(3)] + [torch.empty((B, H, L // w.C, d), **f32)]
    dQr = torch.empty((B, H, L, d), **f32) if rq else None
    klm_lf = torch.empty_like(x["Klm"]) if lf else None
    klm_ml = torch.stack([x["K"][:, :, ::w.C], x["K"][:, :, w.C - 1::w.C]], dim=3).contiguous() if ml else None
    dklm_ml = torch.empty((B, H, L // w.C, 2, d), **f32) if ml else None
    if ml:
        wsf = torch.empty(hils.workspace_size(hils.OP_FWD_ML, w.B, w.H, w.L, w.d, w.C, w.k), dtype=torch.uint8,
                          device="cuda:0")
    import ctypes

    lib = hils._lib
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def step():
        s_ = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        scale = 1.0 / math.sqrt(d)
        if ml:
            hils._check(lib.hils_sparse_attn_fwd_ml(P(x["Q"]), None, P(x["K"]), P(x["V"]), P(klm_ml), 2, P(idx), P(sel),
                                                    1, P(O), P(wt), P(lse), B, H, L, d, w.C, w.k, scale, 0, P(wsf),
                                                    wsf.numel(), s_))
            hils._check(lib.hils_sparse_attn_bwd_ml(P(x["Q"]), None, P(x["K"]), P(x["V"]), P(klm_ml), 2, P(x["dO"]),
                                                    P(idx), P(wt), P(lse), P(grads[0]), None, P(grads[1]),
                                                    P(grads[2]), P(dklm_ml), B, H, L, d, w.C, w.k, scale, 0, P(wsb),
                                                    wsb.numel(), s_))
            return
        if lf:
            qr = P(x["Q_ret"]) if rq else None
            hils._check(lib.hils_sparse_attn_fwd_lf(P(x["Q"]), qr, P(x["K"]), P(x["V"]), P(klm_lf), P(idx), P(sel), 1,
                                                    P(O), P(wt), P(lse), B, H, L, d, w.C, w.k, scale, 0, P(wsf),
                                                    wsf.numel(), s_))
            hils._check(lib.hils_sparse_attn_bwd_lf(P(x["Q"]), qr, P(x["K"]), P(x["V"]), P(klm_lf), P(x["dO"]), P(idx),
                                                    P(wt), P(lse), P(grads[0]), P(dQr) if rq else None,
                                                    *(P(g_) for g_ in grads[1:]), B, H, L, d, w.C, w.k, scale, 0,
                                                    P(wsb), wsb.numel(), s_))
            return
        if not rq:
            hils._check(lib.hils_sparse_attn_fwd(P(x["Q"]), P(x["K"]), P(x["V"]), P(x["Klm"]), P(idx), P(sel), 1,
                                                 P(O), P(wt), P(lse), B, H, L, d, w.C, w.k, scale, 0, P(wsf),
                                                 wsf.numel(), s_))
            hils._check(lib.hils_sparse_attn_bwd(P(x["Q"]), P(x["K"]), P(x["V"]), P(x["Klm"]), P(x["dO"]), P(idx),
                                                 P(wt), P(lse), *(P(g_) for g_ in grads), B, H, L, d, w.C, w.k,
                                                 scale, 0, P(wsb), wsb.numel(), s_))
            return
        hils._check(lib.hils_sparse_attn_fwd_rq(P(x["Q"]), P(x["Q_ret"]), P(x["K"]), P(x["V"]), P(x["Klm"]), P(idx),
                                                P(sel), 1, P(O), P(wt), P(lse), B, H, L, d, w.C, w.k, scale, 0,
                                                P(wsf), wsf.numel(), s_))
        hils._check(lib.hils_sparse_attn_bwd_rq(P(x["Q"]), P(x["Q_ret"]), P(x["K"]), P(x["V"]), P(x["Klm"]),
                                                P(x["dO"]), P(idx), P(wt), P(lse), P(grads[0]), P(dQr),
                                                *(P(g_) for g_ in grads[1:]), B, H, L, d, w.C, w.k, scale, 0,
                                                P(wsb), wsb.numel(), s_))

    ms_eager, _ = timed(step, steps, warmup)
    ms, wall, graph = timed_graph(step, steps, warmup)
    del graph
    nsteps = max(1, min(steps, 10))
    kt = kernel_times(hils, step, nsteps)
    work = train_work(w.B, w.H, w.L, w.d, w.k, w.C)
    res = {
        "tokens_per_s": w.B * w.L / (ms * 1e-3),
        "ms_per_step": ms,
        "ms_per_step_eager": ms_eager,
        "timing": "HIP graph of one step, replayed",
        "wall_s": wall,
        "step_roofline": step_fractions(work, ms),
        "algorithmic_gflop": work["flops"] / 1e9,
        "algorithmic_mb": work["bytes"] / 1e6,
        "kernel_us": {n: round(t / c * 1e3, 3) for n, (t, c) in kt.items()},
        "roofline": roofline(kt, work, {n: c // nsteps for n, (t, c) in kt.items()},
                             None if rq or lf or ml else name),
        "config": {"workload": name, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "C": w.C, "k": w.k,
                   "step": "forward + backward", **({"retrieval_query": True} if rq else {}),
                   **({"landmark_free": True} if lf else {}), **({"landmarks_per_chunk": 2} if ml else {})},
    }
    del x, wsf, wsb
    torch.cuda.empty_cache()
    return res


def bench_decode(hils, synth, name, replicas, warmup, lf=False, ml=False, eager_steps=0):
    """lf: landmark-free chunks; each replica's landmark rows start as its chunks' key means and the step
    maintains the open chunk's row.  eager_steps > 0: run only that many steps of every replica, launched
    one by one without a HIP graph (for counter collection, whose per-dispatch bookkeeping does not cope
    with a graph of thousands of kernel nodes), and return the wall time per token."""
    import torch

    w = synth.WORKLOADS[name]
    x = synth.torch_decode_inputs(w, replicas=replicas)
    reps = x["replicas"]
    if lf:
        for r in reps:
            hils.chunk_means(r["K_cache"], w.C, n_chunks=w.L // w.C, K_lm=r["Klm"])
    if ml:
        # two landmarks per chunk: the given row and a second N(0,1) row
        g = torch.Generator(device="cuda:0")
        g.manual_seed(w.seed + 7)
        for r in reps:
            extra_lm = torch.randn(r["Klm"].shape, generator=g, device="cuda:0").to(r["Klm"].dtype)
            r["Klm"] = torch.stack([r["Klm"], extra_lm], dim=3).contiguous()
    B, H, d = w.B, w.H, w.d
    Lmax = w.L + w.steps
    ws = torch.empty(hils.workspace_size(hils.OP_DECODE, B, H, Lmax, d, w.C, w.k), dtype=torch.uint8,
                     device="cuda:0")
    o = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda:0")
    idx = torch.empty((B, H, w.k + 1), dtype=torch.int32, device="cuda:0")
    wt = torch.empty((B, H, w.k + 1), dtype=torch.float32, device="cuda:0")

    def token(s):
        for r in reps:
            hils.decode_step(x["q"][s], x["k_new"][s], x["v_new"][s], r["K_cache"], r["V_cache"], r["Klm"],
                             w.L + s, w.k, ws=ws, out=o, idx=idx, w=wt, landmark_free=lf)

    for s in range(warmup):
        token(s)
    torch.cuda.synchronize()
    if eager_steps:
        t0 = time.perf_counter()
        for s in range(eager_steps):
            token(s)
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) * 1e6 / (eager_steps * len(reps))
        del x, reps, ws
        torch.cuda.empty_cache()
        return {"us_per_token_eager": us, "timing": f"{eager_steps} steps per replica, launched eagerly",
                "config": {"workload": name, "B": B, "H": H, "d": d, "context": w.L, "steps": eager_steps,
                           "k": w.k, "replicas": replicas, **({"landmark_free": True} if lf else {}),
                           **({"landmarks_per_chunk": 2} if ml else {})}}
    # eager pass (host launch overhead included), then the whole run captured once and replayed
    t0 = time.perf_counter()
    for s in range(w.steps):
        token(s)
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - t0) * 1e6 / (w.steps * len(reps))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in range(w.steps):
            token(s)
    graph.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(st)
    graph.replay()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del graph
    calls = w.steps * len(reps)
    us = e0.elapsed_time(e1) * 1e3 / calls
    # per-step distribution: each step (all replicas) in a graph of its own, replayed once untimed and once
    # timed; re-running a step rewrites the same cache rows, and later rows are not read by it
    step_us = []
    # (one replica: a step's graph would hold three kernels and its launch cost would set the figure)
    for s in range(w.steps if len(reps) > 1 else 0):
        gs = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gs):
            token(s)
        gs.replay()
        e0.record(st)
        gs.replay()
        e1.record(st)
        torch.cuda.synchronize()
        step_us.append(e0.elapsed_time(e1) * 1e3 / len(reps))
        del gs
    step_us.sort()
    # per-kernel times over a further pass of 4 tokens, enqueued while the GPU is busy
    hils.profile_enable(True)
    host_ahead()
    for s in range(4):
        token(s)
    torch.cuda.synchronize()
    kt = hils.profile_read()
    hils.profile_enable(False)
    mid = w.L + w.steps // 2
    work = decode_work(B, H, d, mid, w.k, w.C)
    res = {
        "us_per_token": us,
        "us_per_token_eager": eager_us,
        "us_per_token_p50": step_us[len(step_us) // 2] if step_us else None,
        "us_per_token_p90": step_us[(9 * len(step_us)) // 10] if step_us else None,
        "timing": "every step of every replica captured in one HIP graph, replayed once; p50 and p90 over the "
                  "steps, each step's replicas in a graph of their own",
        "hbm_gbs": work["bytes"] / (us * 1e-6) / 1e9,
        "hbm_frac": work["bytes"] / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
        "step_roofline": step_fractions(work, us * 1e-3),
        "bytes_per_token": work["bytes"],
        "calls": calls,
        "wall_s": wall,
        # each kernel bracketed by HIP events on its stream: for kernels of a few microseconds the bracket adds
        # the launch's dispatch latency, so these exceed the kernels' own durations (rocprofv3 gives those)
        "kernel_us": {n: round(t / c * 1e3, 3) for n, (t, c) in kt.items()},
        "roofline": roofline(kt, work, {n: 1 for n in kt}, None if lf or ml else name, by_bytes=True),
        "config": {"workload": name, "B": B, "H": H, "d": d, "context": w.L, "steps": w.steps, "k": w.k,
                   "replicas": len(reps), "protocol": "cold" if len(reps) > 1 else "warm",
                   **({"landmark_free": True} if lf else {}), **({"landmarks_per_chunk": 2} if ml else {})},
    }
    del x, reps, ws
    torch.cuda.empty_cache()
    return res


def bench_decode_paged(hils, synth, name, warmup):
    """Batched decode of ragged sequences over a paged cache: one step advances every sequence by one token."""
    import torch

    w = synth.WORKLOADS[name]
    x = synth.torch_paged_decode_inputs(w)
    B, H, d = w.B, w.H, w.d
    maxp = x["page_table"].shape[1]
    ws = torch.empty(hils.workspace_size(hils.OP_DECODE, B, H, maxp * w.C, d, w.C, w.k), dtype=torch.uint8,
                     device="cuda:0")
    o = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda:0")
    idx = torch.empty((B, H, w.k + 1), dtype=torch.int32, device="cuda:0")
    wt = torch.empty((B, H, w.k + 1), dtype=torch.float32, device="cuda:0")

    def step(s):
        hils.decode_step_paged(x["q"][s], x["k_new"][s], x["v_new"][s], x["K_pages"], x["V_pages"], x["K_lm_pages"],
                               x["page_table"], x["pos"][s], x["pos_max"][s], w.k, ws=ws, out=o, idx=idx, w=wt)

    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in range(w.steps):
            step(s)
    graph.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    graph.replay()
    e1.record(st)
    torch.cuda.synchronize()
    del graph
    us = e0.elapsed_time(e1) * 1e3 / w.steps
    hils.profile_enable(True)
    host_ahead()
    for s in range(8):
        step(s)
    torch.cuda.synchronize()
    kt = hils.profile_read()
    hils.profile_enable(False)
    # landmark rows read per step (every sequence scans its chunks) and the kept chunks' keys and values
    lm_bytes = sum(c // w.C for c in x["ctx"]) * H * d * 2
    kv_bytes = B * H * (w.k + 1) * w.C * d * 2 * 2
    res = {
        "us_per_step": us,
        "tokens_per_s": B / (us * 1e-6),
        "timing": "every step captured in one HIP graph, replayed once",
        "hbm_gbs": (lm_bytes + kv_bytes) / (us * 1e-6) / 1e9,
        "kernel_us": {n: round(t / c * 1e3, 3) for n, (t, c) in kt.items()},
        "config": {"workload": name, "B": B, "H": H, "d": d, "contexts": [min(x["ctx"]), max(x["ctx"])],
                   "steps": w.steps, "k": w.k, "pages": int(x["K_pages"].shape[0]), "cache": "paged, page = chunk"},
    }
    del x, ws
    torch.cuda.empty_cache()
    return res


def _threads():
    return len(os.sched_getaffinity(0))


def cpu_baseline(synth, name):
    """The oracle (plain C, double precision) on the host cores, on the full 8K workload."""
    import oracle

    w = synth.WORKLOADS[name]
    x = synth.workload_inputs(w)
    nthreads = _threads()
    # the full forward, repeated until about ten seconds of host work have run (at most 40 passes)
    reps, dt = 0, 0.0
    while reps < 40 and (reps == 0 or dt < 10.0):
        t0 = time.perf_counter()
        r = oracle.fwd(x["Q"], x["K"], x["V"], x["Klm"], w.C, w.k, nthreads=nthreads)
        dt += time.perf_counter() - t0
        reps += 1
    return {"value": reps * w.B * w.L / dt, "unit": "tokens/s", "cores": int(r["threads"]), "kind": "oracle",
            "sample": f"full {name} forward (B={w.B} H={w.H} L={w.L} d={w.d} k={w.k}) x {reps}, {dt:.1f} s"}


def cpu_baseline_prefill_heads(synth, name, heads):
    """The oracle's forward on ``heads`` of the workload's H heads (same shapes per head), scaled to all
    heads: the work is exactly linear in the head count."""
    import oracle

    w = synth.WORKLOADS[name]
    x = synth.workload_inputs(w, H=heads)
    t0 = time.perf_counter()
    r = oracle.fwd(x["Q"], x["K"], x["V"], x["Klm"], w.C, w.k, nthreads=_threads())
    dt = time.perf_counter() - t0
    scale = w.H / heads
    return {"value": w.B * w.L / (dt * scale), "unit": "tokens/s", "cores": int(r["threads"]), "kind": "oracle",
            "sample": f"{name} forward on {heads} of {w.H} heads (B={w.B} L={w.L} d={w.d} k={w.k}), {dt:.1f} s, "
                      f"scaled x{scale:g} to all heads"}


def cpu_baseline_decode(synth, name, heads, steps):
    """The oracle's decode steps on ``heads`` of the workload's heads at its context, scaled to all heads."""
    import oracle

    w = synth.WORKLOADS[name]
    x = synth.workload_inputs(w, H=heads, steps=steps)
    Kc, Vc = x["K_cache"], x["V_cache"]
    nthreads = _threads()
    t0 = time.perf_counter()
    for s in range(steps):
        r = oracle.decode(x["q"][s], x["k_new"][s], x["v_new"][s], Kc, Vc, x["Klm"], w.L + s, w.C, w.k,
                          nthreads=nthreads)
    dt = time.perf_counter() - t0
    scale = w.H / heads
    return {"value": dt / steps * scale * 1e6, "unit": "us/token", "cores": int(r["threads"]), "kind": "oracle",
            "sample": f"{name}: {steps} decode steps on {heads} of {w.H} heads at context {w.L} (d={w.d} k={w.k}), "
                      f"{dt:.1f} s, scaled x{scale:g} to all heads"}


def cpu_baseline_train(synth, name, batch):
    """The oracle's forward and backward (selection from its forward) on ``batch`` of the workload's B
    sequences, scaled to the whole batch."""
    import oracle

    w = synth.WORKLOADS[name]
    x = synth.workload_inputs(w, B=batch, with_dO=True)
    nthreads = _threads()
    t0 = time.perf_counter()
    f = oracle.fwd(x["Q"], x["K"], x["V"], x["Klm"], w.C, w.k, nthreads=nthreads)
    oracle.bwd(x["Q"], x["K"], x["V"], x["Klm"], x["dO"], f["idx"], w.C, w.k, nthreads=nthreads)
    dt = time.perf_counter() - t0
    scale = w.B / batch
    return {"value": w.B * w.L / (dt * scale), "unit": "tokens/s", "cores": int(f["threads"]), "kind": "oracle",
            "sample": f"{name} forward + backward on {batch} of {w.B} sequences (H={w.H} L={w.L} d={w.d} k={w.k}), "
                      f"{dt:.1f} s, scaled x{scale:g} to the whole batch"}


def measured_peaks():
    """Rates the box reaches with library kernels: a 1 GiB device copy (HBM read + write) and a bf16
    8192^3 matrix product (hipBLASLt on MFMA).  Context for the spec peaks the rooflines use."""
    import torch

    out = {}
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    out["hbm_copy_GBs"] = round(2 * nbytes * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del src, dst
    n = 8192
    a = torch.randn((n, n), device="cuda:0", dtype=torch.bfloat16)
    b = torch.randn((n, n), device="cuda:0", dtype=torch.bfloat16)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    out["bf16_gemm_TFLOPs"] = round(2 * n ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    del a, b, c
    torch.cuda.empty_cache()
    out["note"] = "1 GiB device copy (read + write bytes) and a bf16 8192^3 torch matmul, 10 runs each"
    return out


# ----------------------------------------------------------------------------- main


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--skip", default="", help="comma list of workloads to skip")
    ap.add_argument("--only", default="", help="run only this workload (prefill_8k, prefill_128k, decode_512k, "
                                               "train_8k; a _retrieval suffix on a prefill or train workload "
                                               "adds separate retrieval queries, a _landmark_free suffix on a "
                                               "prefill, decode or train workload uses key-mean landmarks, a "
                                               "_two_landmarks suffix on a prefill, train or decode workload uses "
                                               "two landmarks per chunk (prefill and train: the "
                                               "first and last token of each chunk) and print "
                                               "its result object; for profiling runs")
    ap.add_argument("--decode-replicas", type=int, default=32)
    ap.add_argument("--decode-eager-steps", type=int, default=0,
                    help="with --only decode_*: run this many steps per replica without a HIP graph (counter runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the HiLS hot path here is built and timed on a single MI355X; "
              "--gpus above 1 is not supported.", file=sys.stderr)
        sys.exit(2)
    import torch

    from long_context_landmark_amd import hils, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    skip = set(s for s in args.skip.split(",") if s)
    torch.cuda.set_device(0)
    if args.only:
        if args.only == "copy_calibration":
            # a plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters
            nbytes = 1 << 30
            src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            print(json.dumps({"workload": "copy_calibration", "bytes_per_copy": nbytes, "copies": 3}), flush=True)
            return
        rq = args.only.endswith("_retrieval")
        lf = args.only.endswith("_landmark_free")
        ml = args.only.endswith("_two_landmarks")
        name = args.only
        for suffix in ("_retrieval", "_landmark_free", "_two_landmarks"):
            if name.endswith(suffix):
                name = name[:-len(suffix)]
        if name.startswith("prefill"):
            res = bench_prefill(hils, synth, name, args.steps, args.warmup, rq=rq, lf=lf, ml=ml)
        elif name.startswith("decode_paged"):
            res = bench_decode_paged(hils, synth, name, args.warmup)
        elif name.startswith("decode"):
            res = bench_decode(hils, synth, name, args.decode_replicas, args.warmup, lf=lf, ml=ml,
                               eager_steps=args.decode_eager_steps)
        elif name.startswith("train"):
            res = bench_train(hils, synth, name, args.steps, args.warmup, rq=rq, lf=lf, ml=ml)
        else:
            raise SystemExit(f"unknown workload {args.only}")
        print(json.dumps({"workload": args.only, **res}), flush=True)
        return
    log(f"[bench] prefill_8k: {args.steps} steps, {args.warmup} warmup")
    head = bench_prefill(hils, synth, "prefill_8k", args.steps, args.warmup)
    log(f"[bench] prefill_8k {head['tokens_per_s']:.4g} tokens/s, {head['ms_per_step']*1e3:.1f} us/step")
    extra = {}
    if "prefill_128k" not in skip:
        log("[bench] prefill_128k")
        extra["prefill_128k"] = bench_prefill(hils, synth, "prefill_128k", max(3, min(args.steps, 10)), 2)
        log(f"[bench] prefill_128k {extra['prefill_128k']['tokens_per_s']:.4g} tokens/s")
    if "decode_512k" not in skip:
        log(f"[bench] decode_512k cold ({args.decode_replicas} replicas)")
        extra["decode_512k"] = bench_decode(hils, synth, "decode_512k", args.decode_replicas, 4)
        log(f"[bench] decode_512k {extra['decode_512k']['us_per_token']:.2f} us/token")
        log("[bench] decode_512k warm (1 replica)")
        extra["decode_512k_warm"] = bench_decode(hils, synth, "decode_512k", 1, 4)
    if "train_8k" not in skip:
        log("[bench] train_8k")
        extra["train_8k"] = bench_train(hils, synth, "train_8k", max(3, min(args.steps, 20)), 2)
        log(f"[bench] train_8k {extra['train_8k']['ms_per_step']*1e3:.1f} us/step")
    if "retrieval" not in skip:
        # separate retrieval queries score the landmarks (low-rank query calibration)
        log("[bench] prefill_8k and train_8k with retrieval queries")
        extra["prefill_8k_retrieval"] = bench_prefill(hils, synth, "prefill_8k", max(3, min(args.steps, 20)), 2,
                                                      rq=True)
        extra["train_8k_retrieval"] = bench_train(hils, synth, "train_8k", max(3, min(args.steps, 20)), 2, rq=True)
        log(f"[bench] prefill_8k_retrieval {extra['prefill_8k_retrieval']['ms_per_step']*1e3:.1f} us/step, "
            f"train_8k_retrieval {extra['train_8k_retrieval']['ms_per_step']*1e3:.1f} us/step")
    if "landmark_free" not in skip:
        # landmark-free chunks: key-mean landmarks formed inside the step (prefill) or by the step (decode)
        log("[bench] prefill_8k and decode_512k with landmark-free chunks")
        extra["prefill_8k_landmark_free"] = bench_prefill(hils, synth, "prefill_8k", max(3, min(args.steps, 20)), 2,
                                                          lf=True)
        extra["decode_512k_landmark_free"] = bench_decode(hils, synth, "decode_512k", args.decode_replicas, 4,
                                                          lf=True)
        extra["train_8k_landmark_free"] = bench_train(hils, synth, "train_8k", max(3, min(args.steps, 20)), 2, lf=True)
        log(f"[bench] prefill_8k_landmark_free {extra['prefill_8k_landmark_free']['ms_per_step']*1e3:.1f} us/step, "
            f"decode_512k_landmark_free {extra['decode_512k_landmark_free']['us_per_token']:.2f} us/token")
    if "two_landmarks" not in skip:
        # two landmarks per chunk (the keys of its first and last token), log-sum-exp chunk scores
        log("[bench] prefill_8k and train_8k with two landmarks per chunk")
        extra["prefill_8k_two_landmarks"] = bench_prefill(hils, synth, "prefill_8k", max(3, min(args.steps, 20)), 2,
                                                          ml=True)
        extra["train_8k_two_landmarks"] = bench_train(hils, synth, "train_8k", max(3, min(args.steps, 20)), 2, ml=True)
        extra["decode_512k_two_landmarks"] = bench_decode(hils, synth, "decode_512k", args.decode_replicas, 4, ml=True)
        log(f"[bench] prefill_8k_two_landmarks {extra['prefill_8k_two_landmarks']['ms_per_step']*1e3:.1f} us/step, "
            f"train_8k_two_landmarks {extra['train_8k_two_landmarks']['ms_per_step']*1e3:.1f} us/step")
    if "decode_paged_b16" not in skip:
        log("[bench] decode_paged_b16 (16 ragged sequences, paged cache)")
        extra["decode_paged_b16"] = bench_decode_paged(hils, synth, "decode_paged_b16", 4)
        log(f"[bench] decode_paged_b16 {extra['decode_paged_b16']['us_per_step']:.2f} us/step")
    log("[bench] measured peaks (library copy and matmul)")
    peaks = measured_peaks()
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle): prefill_8k")
        cpu = cpu_baseline(synth, "prefill_8k")
        if "prefill_128k" in extra:
            log("[bench] cpu baseline (oracle): prefill_128k, 2 heads")
            extra["prefill_128k"]["cpu_baseline"] = cpu_baseline_prefill_heads(synth, "prefill_128k", 2)
        if "decode_512k" in extra:
            log("[bench] cpu baseline (oracle): decode_512k, 4 heads, 64 steps")
            extra["decode_512k"]["cpu_baseline"] = cpu_baseline_decode(synth, "decode_512k", 4, 64)
        if "train_8k" in extra:
            log("[bench] cpu baseline (oracle): train_8k, 1 sequence")
            extra["train_8k"]["cpu_baseline"] = cpu_baseline_train(synth, "train_8k", 1)
    line = {
        "metric": METRIC,
        "value": round(head["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "measured_peaks": peaks,
        "detail": {"prefill_8k": {k: v for k, v in head.items() if k not in ("roofline", "config")}},
        "workloads": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
