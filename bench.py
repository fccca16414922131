#!/usr/bin/env python3
"""Benchmark of the Parallax operator on one MI355X.

Headline (``value``): causal GQA prefill in bf16 with fp32 accumulation,
B=4, Hq=16, Hkv=8, T=4096, d=128, rho = W_R x, in TFLOP/s over the method's
four causal GEMM-equivalents (QK, rho K, PV, (P.R)V: 2*d flops per (i, j<=i)
pair each).  The same JSON line also carries the decode workloads (batched
B=64 ctx=8192, and long-context ragged B=8 ctx ~ U{16384..131072}) in
microseconds per step and HBM GB/s, and the training step (forward + backward,
B=8 T=4096) in TFLOP/s per pass.

Timing: HIP events recorded on the stream the kernels run on (torch's current
stream), W warm-up steps, then exactly K timed steps between two device
synchronisations.  The CPU baseline is the fp64 oracle on a bounded sample of
prefill rows, timed on the host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--only all|prefill|decode|decode_long|train|copy|decode_sweep] [--no-cpu] [--no-graph]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill TFLOP/s & %MFMA peak; decode µs/step & HBM GB/s vs peak"
PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 / fp16 MFMA (no sparsity)
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The GPU raises its clocks only under sustained work (about 40 ms on the
# MI355X measured here: the prefill takes 790 us cold and 520 us warm), so
# every timed region is preceded by at least this much back-to-back work on
# top of the requested warm-up steps.
CLOCK_WARM_MS = 60.0


def warm_clocks(fn, ms=CLOCK_WARM_MS):
    """Run fn back to back, with no host synchronisation in between, for at
    least ``ms`` of device time (the per-call time is estimated from a short
    probe first, so short calls are not separated by idle gaps)."""
    import torch

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    fn()
    start.record()
    for _ in range(4):
        fn()
    stop.record()
    stop.synchronize()
    per_call = max(start.elapsed_time(stop) / 4, 1e-3)
    n = int(math.ceil(1.5 * ms / per_call))  # the probe ran at cold clocks: overshoot
    for _ in range(n):
        fn()
    torch.cuda.synchronize()
    return n + 5


def time_steps(fn, steps, warmup):
    """Average ms per call of fn over `steps` timed calls (after a clock
    warm-up of at least CLOCK_WARM_MS and `warmup` further calls)."""
    import torch

    warm_clocks(fn)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def time_graph_steps(fn, per_graph, replays, warmup):
    """Average ms per call of fn when `per_graph` calls are captured in one HIP
    graph and the graph is replayed `replays` times (launch gaps removed)."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            fn()
    ms = time_steps(graph.replay, replays, warmup)
    del graph
    return ms / per_graph


def causal_pairs(T):
    return T * (T + 1) // 2


# ------------------------------------------------------------------ prefill
def bench_prefill(steps, warmup):
    import torch

    from parallax_local_linear_plx_amd import inputs, plx_fwd_prefill

    B, Hq, Hkv, T, d = 4, 16, 8, 4096, 128
    q = inputs.device_normal((B, Hq, T, d), 1.0, 21)
    k = inputs.device_normal((B, Hkv, T, d), 1.0, 22)
    v = inputs.device_normal((B, Hkv, T, d), 1.0, 23)
    rho = inputs.device_projected_probe(B, Hq, T, d, 24)
    o = torch.empty((B, Hq, T, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")

    def step():
        plx_fwd_prefill(q, k, v, rho, o=o, lse=True)

    ms = time_steps(step, steps, warmup)
    flops = 4 * 2 * d * causal_pairs(T) * B * Hq
    tflops = flops / (ms * 1e-3) / 1e12
    # bytes the kernel must move at least once: q, rho, k, v in; o, lse out
    algo_bytes = (2 * B * Hq * T * d + 2 * B * Hkv * T * d) * 2 + B * Hq * T * (d + 1) * 4
    cfg = {"workload": f"bf16 causal GQA prefill B={B} Hq={Hq} Hkv={Hkv} T={T} d={d}, rho=W_R x",
           "B": B, "Hq": Hq, "Hkv": Hkv, "T": T, "d": d}
    return {"ms": ms, "tflops": tflops, "flops": flops, "bytes": algo_bytes, "config": cfg}


# ------------------------------------------------------------------- decode
def bench_decode(steps, warmup, B, ctx_len, S_max, name, seed, graph=True, Hq=16, Hkv=8):
    import torch

    from parallax_local_linear_plx_amd import inputs, plx_decode

    d = 128
    kc = inputs.device_normal((B, Hkv, S_max, d), 1.0, seed)
    vc = inputs.device_normal((B, Hkv, S_max, d), 1.0, seed + 1)
    q = inputs.device_normal((B, Hq, d), 1.0, seed + 2)
    rho = inputs.device_normal((B, Hq, d), 0.1, seed + 3)
    ctx = torch.from_numpy(np.asarray(ctx_len, np.int32)).cuda()
    o = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    from parallax_local_linear_plx_amd import decode_workspace_size

    ws = torch.empty(decode_workspace_size(B, Hq, Hkv, S_max, d, 0), dtype=torch.uint8, device="cuda")

    def step():
        plx_decode(q, rho, kc, vc, ctx, num_splits=0, workspace=ws, o=o, lse=False)

    ms = time_steps(step, steps, warmup)
    # the same steps captured ten to a graph, as a serving loop would replay them
    ms_graph = time_graph_steps(step, 10, max(1, steps // 10), max(1, warmup // 10)) if graph else None
    kv_bytes = int(np.sum(ctx_len)) * Hkv * d * 2 * 2
    io_bytes = B * Hq * d * (2 + 2 + 4)
    gbs = (kv_bytes + io_bytes) / (ms * 1e-3) / 1e9
    flops = int(np.sum(ctx_len)) * Hq * d * 8
    del kc, vc
    torch.cuda.empty_cache()
    return {"workload": name, "us_per_step": ms * 1e3, "us_per_token": ms * 1e3,
            "GB/s": gbs, "hbm_frac": gbs / PEAK_HBM_GBS, "bytes": kv_bytes + io_bytes,
            "us_per_step_graph10": ms_graph * 1e3 if graph else None,
            "GB/s_graph10": (kv_bytes + io_bytes) / (ms_graph * 1e-3) / 1e9 if graph else None,
            "flop_per_byte": flops / (kv_bytes + io_bytes),
            "ctx_len_sum": int(np.sum(ctx_len))}


# ------------------------------------------------------------ decode sweep
SWEEP_BATCH = (1, 4, 16, 64, 128)
SWEEP_CTX = (1024, 4096, 16384, 65536, 131072)
SWEEP_MAX_KEYS = 1 << 22  # B * ctx cap: 17 GB of K and V


def bench_decode_sweep(steps, warmup):
    """Decode latency over batch x context (uniform lengths), automatic schedule.
    One K/V buffer sized for the largest cell is filled once and viewed per cell."""
    import torch

    from parallax_local_linear_plx_amd import decode_workspace_size, plx_decode

    Hq, Hkv, d = 16, 8, 128
    n = SWEEP_MAX_KEYS * Hkv * d
    g = torch.Generator(device="cuda")
    g.manual_seed(51)
    kv = []
    for _ in range(2):
        buf = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        chunk = 1 << 26
        for i in range(0, n, chunk):
            m = min(chunk, n - i)
            buf[i:i + m] = torch.randn(m, generator=g, device="cuda").to(torch.bfloat16)
        kv.append(buf)
    cells = []
    for B in SWEEP_BATCH:
        for ctx in SWEEP_CTX:
            if B * ctx > SWEEP_MAX_KEYS:
                continue
            kc = kv[0][:B * Hkv * ctx * d].view(B, Hkv, ctx, d)
            vc = kv[1][:B * Hkv * ctx * d].view(B, Hkv, ctx, d)
            q = torch.randn(B, Hq, d, generator=g, device="cuda").to(torch.bfloat16)
            rho = (0.1 * torch.randn(B, Hq, d, generator=g, device="cuda")).to(torch.bfloat16)
            cl = torch.full((B,), ctx, dtype=torch.int32, device="cuda")
            o = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
            ws = torch.empty(decode_workspace_size(B, Hq, Hkv, ctx, d, 0), dtype=torch.uint8, device="cuda")

            def step():
                plx_decode(q, rho, kc, vc, cl, num_splits=0, workspace=ws, o=o, lse=False)

            ms = time_steps(step, steps, warmup)
            # ten calls to a graph: the device time without the host's launch path
            msg = time_graph_steps(step, 10, max(2, steps // 10), 1)
            nbytes = B * Hkv * ctx * d * 2 * 2 + B * Hq * d * (2 + 2 + 4)
            gbs = nbytes / (ms * 1e-3) / 1e9
            gbsg = nbytes / (msg * 1e-3) / 1e9
            cells.append({"B": B, "ctx": ctx, "us_per_step": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
                          "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                          "us_per_step_graph10": round(msg * 1e3, 2), "GB/s_graph10": round(gbsg, 1),
                          "hbm_frac_graph10": round(gbsg / PEAK_HBM_GBS, 4)})
            log(f"  B={B:4d} ctx={ctx:7d}: {ms * 1e3:9.1f} us  {gbs:7.0f} GB/s  ({gbs / PEAK_HBM_GBS:.1%})"
                f"   graph: {msg * 1e3:9.1f} us  {gbsg:7.0f} GB/s  ({gbsg / PEAK_HBM_GBS:.1%})")
    return {"workload": "bf16 decode sweep Hq=16 Hkv=8 d=128, uniform ctx, automatic schedule",
            "cells": cells}


# ------------------------------------------------------------------ training
def bench_train(steps, warmup):
    import torch

    from parallax_local_linear_plx_amd import bwd_workspace_size, inputs, plx_bwd, plx_fwd_prefill

    B, Hq, Hkv, T, d = 8, 16, 8, 4096, 128
    q = inputs.device_normal((B, Hq, T, d), 1.0, 51)
    k = inputs.device_normal((B, Hkv, T, d), 1.0, 52)
    v = inputs.device_normal((B, Hkv, T, d), 1.0, 53)
    rho = inputs.device_normal((B, Hq, T, d), 0.1, 54)
    d_o = inputs.device_normal((B, Hq, T, d), 1.0, 55)
    fwd = plx_fwd_prefill(q, k, v, rho, aux=True)
    ws = torch.empty(bwd_workspace_size(B, Hq, Hkv, T, d), dtype=torch.uint8, device="cuda")
    grads = {
        "dq": torch.empty_like(fwd["o"]), "drho": torch.empty_like(fwd["o"]),
        "dk": torch.empty((B, Hkv, T, d), dtype=torch.float32, device="cuda"),
        "dv": torch.empty((B, Hkv, T, d), dtype=torch.float32, device="cuda"),
    }

    def fstep():
        plx_fwd_prefill(q, k, v, rho, o=fwd["o"], aux=True)

    def bstep():
        plx_bwd(q, k, v, rho, d_o, fwd["o"], fwd["lse"], fwd["c"], fwd["vbar"], workspace=ws, grads=grads)

    ms_f = time_steps(fstep, steps, warmup)
    ms_b = time_steps(bstep, steps, warmup)
    fl_f = 4 * 2 * d * causal_pairs(T) * B * Hq
    fl_b = 8 * 2 * d * causal_pairs(T) * B * Hq
    out = {"workload": f"bf16 training step fwd+bwd B={B} Hq={Hq} Hkv={Hkv} T={T} d={d}",
           "fwd_ms": ms_f, "bwd_ms": ms_b, "step_ms": ms_f + ms_b,
           "fwd_tflops": fl_f / (ms_f * 1e-3) / 1e12, "bwd_tflops": fl_b / (ms_b * 1e-3) / 1e12,
           "step_tflops": (fl_f + fl_b) / ((ms_f + ms_b) * 1e-3) / 1e12, "bwd_flops": fl_b}
    out["bwd_mfma_frac"] = out["bwd_tflops"] / PEAK_BF16_TFLOPS
    del q, k, v, rho, d_o, fwd, grads
    torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------- projection
def bench_proj(steps, warmup):
    """The stacked [W_Q; W_K; W_V; W_R] projection of the prefill workload's
    layer (B=4, T=4096, D=1024 -> Hq=16, Hkv=8, d=128).  torch.matmul of the
    same shapes (a library GEMM writing one [B T, N] matrix, no head-major
    scatter) is timed beside it for context."""
    import torch

    from parallax_local_linear_plx_amd import inputs, plx_qkvr_proj

    B, T, D, Hq, Hkv, d = 4, 4096, 1024, 16, 8, 128
    N = (2 * Hq + 2 * Hkv) * d
    x = inputs.device_normal((B, T, D), 1.0, 61)
    w = inputs.device_normal((N, D), 1.0 / np.sqrt(D), 62)
    out = plx_qkvr_proj(x, w, Hq, Hkv, d)

    def step():
        plx_qkvr_proj(x, w, Hq, Hkv, d, out=out)

    ms = time_steps(step, steps, warmup)
    x2, wt = x.view(B * T, D), w.t()
    y = torch.empty((B * T, N), dtype=torch.bfloat16, device="cuda")
    ms_lib = time_steps(lambda: torch.matmul(x2, wt, out=y), steps, warmup)
    flops = 2 * B * T * N * D
    algo_bytes = (B * T * D + N * D + B * T * N) * 2
    tf = flops / (ms * 1e-3) / 1e12
    del x, w, out, y
    torch.cuda.empty_cache()
    return {"workload": f"bf16 stacked projection [Q|K|V|rho] = x W^T, B={B} T={T} D={D} "
                        f"Hq={Hq} Hkv={Hkv} d={d} (N={N}), head-major outputs",
            "us_per_call": ms * 1e3, "tflops": tf, "flops": flops, "bytes": algo_bytes,
            "library_matmul_us": ms_lib * 1e3,
            "library_matmul_tflops": flops / (ms_lib * 1e-3) / 1e12,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": measured_traffic("proj"), "kernel": "proj_kernel",
                         "algorithmic_flops_per_launch": flops}}


# ------------------------------------------------------- head-dim variants
def bench_headdim(steps, warmup):
    """Prefill and backward (B=4, Hq=16, Hkv=8, T=4096) and decode (B=64,
    Hq=16, Hkv=8, ctx=8192) at d = 64 and d = 256, for comparison with the
    d = 128 lines."""
    import torch

    from parallax_local_linear_plx_amd import (bwd_workspace_size, decode_workspace_size, inputs, plx_bwd,
                                               plx_decode, plx_fwd_prefill)

    out = {}
    for d in (64, 256):
        B, Hq, Hkv, T = 4, 16, 8, 4096
        q = inputs.device_normal((B, Hq, T, d), 1.0, 71)
        k = inputs.device_normal((B, Hkv, T, d), 1.0, 72)
        v = inputs.device_normal((B, Hkv, T, d), 1.0, 73)
        rho = inputs.device_normal((B, Hq, T, d), 0.1, 74)
        o = torch.empty((B, Hq, T, d), dtype=torch.float32, device="cuda")
        ms = time_steps(lambda: plx_fwd_prefill(q, k, v, rho, o=o, lse=True), steps, warmup)
        flops = 4 * 2 * d * causal_pairs(T) * B * Hq
        # backward of the same shape (dO ~ N(0, 1))
        d_o = inputs.device_normal((B, Hq, T, d), 1.0, 79)
        fwd = plx_fwd_prefill(q, k, v, rho, aux=True)
        ws_b = torch.empty(bwd_workspace_size(B, Hq, Hkv, T, d), dtype=torch.uint8, device="cuda")
        grads = {"dq": torch.empty_like(fwd["o"]), "drho": torch.empty_like(fwd["o"]),
                 "dk": torch.empty((B, Hkv, T, d), dtype=torch.float32, device="cuda"),
                 "dv": torch.empty((B, Hkv, T, d), dtype=torch.float32, device="cuda")}
        ms_b = time_steps(lambda: plx_bwd(q, k, v, rho, d_o, fwd["o"], fwd["lse"], fwd["c"], fwd["vbar"],
                                          workspace=ws_b, grads=grads), steps, warmup)
        del q, k, v, rho, o, d_o, fwd, ws_b, grads
        Bd, S = 64, 8192
        qd = inputs.device_normal((Bd, Hq, d), 1.0, 75)
        rd = inputs.device_normal((Bd, Hq, d), 0.1, 76)
        kc = inputs.device_normal((Bd, Hkv, S, d), 1.0, 77)
        vc = inputs.device_normal((Bd, Hkv, S, d), 1.0, 78)
        ctx = torch.full((Bd,), S, dtype=torch.int32, device="cuda")
        ws = torch.empty(decode_workspace_size(Bd, Hq, Hkv, S, d, 0), dtype=torch.uint8, device="cuda")
        od = torch.empty((Bd, Hq, d), dtype=torch.float32, device="cuda")
        msd = time_steps(lambda: plx_decode(qd, rd, kc, vc, ctx, num_splits=0, workspace=ws, o=od), steps, warmup)
        nbytes = Bd * Hkv * S * d * 4 + Bd * Hq * d * 8
        del qd, rd, kc, vc, ws, od
        torch.cuda.empty_cache()
        out[f"d{d}"] = {"prefill_us": ms * 1e3, "prefill_tflops": flops / (ms * 1e-3) / 1e12,
                        "prefill_mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                        "bwd_us": ms_b * 1e3, "bwd_tflops": 2 * flops / (ms_b * 1e-3) / 1e12,
                        "bwd_mfma_frac": 2 * flops / (ms_b * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                        "decode_us": msd * 1e3, "decode_GB/s": nbytes / (msd * 1e-3) / 1e9,
                        "decode_hbm_frac": nbytes / (msd * 1e-3) / 1e9 / PEAK_HBM_GBS}
    return out


# ------------------------------------------------------- measured ceilings
def measured_peaks(reps=10):
    """Ceilings measured on this GPU, reported beside the published peaks:
    the bf16 rate of independent 16x16x32 MFMA chains with nothing else in the
    loop (1024 workgroups of four waves), and the best HBM read rate of a
    streaming kernel (32 KB tiles, eight 16-byte loads in flight per thread,
    1024 to 8192 workgroups) over a 2 GiB buffer, above the 256 MB last-level
    cache.  Both kernels live in libplx_peak.so."""
    import ctypes

    import torch

    path = os.path.join(ROOT, "parallax_local_linear_plx_amd", "libplx_peak.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with python -m parallax_local_linear_plx_amd.build")
    L = ctypes.CDLL(path)
    L.plx_peak_mfma_flops.restype = ctypes.c_double
    L.plx_peak_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    L.plx_peak_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.plx_peak_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = torch.empty(4096, dtype=torch.float32, device="cuda")

    def best_ms(fn):
        # the same sustained warm-up as every timed leg, so the ceiling is
        # taken at the clocks the kernels run at
        warm_clocks(fn)
        ts = []
        for _ in range(reps):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            torch.cuda.synchronize()
            ts.append(s.elapsed_time(e))
        return min(ts)

    blocks, iters = 1024, 4000  # about a millisecond per launch

    def mfma():
        if L.plx_peak_mfma_bf16(ctypes.c_void_p(out.data_ptr()), blocks, iters, stream) != 0:
            raise RuntimeError("plx_peak_mfma_bf16 failed")
    tflops = L.plx_peak_mfma_flops(blocks, iters) / (best_ms(mfma) * 1e-3) / 1e12
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    gbs = 0.0
    for nb in (1024, 2048, 4096, 8192):
        def read(nb=nb):
            if L.plx_peak_hbm_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(out.data_ptr()),
                                   nb, stream) != 0:
                raise RuntimeError("plx_peak_hbm_read failed")
        gbs = max(gbs, nbytes / (best_ms(read) * 1e-3) / 1e9)
    del buf
    return {"mfma_bf16_tflops": round(tflops, 1), "hbm_read_gbs": round(gbs, 1),
            "mfma_kernel": "mfma_peak_kernel: 8 independent v_mfma_f32_16x16x32_bf16 chains per wave",
            "hbm_kernel": "hbm_read_kernel: 32 KB tiles of 16-byte loads over 2 GiB"}


# -------------------------------------------------------- copy calibration
def bench_copy(steps, nbytes=1 << 30):
    """A plain device-to-device copy of a known size.  Run under rocprofv3
    --pmc FETCH_SIZE / WRITE_SIZE, it gives the factor between those counters
    and true bytes on this GPU, which scales the kernels' counter readings."""
    import torch

    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ms = time_steps(lambda: dst.copy_(src), steps, 1)
    return {"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "ms": ms,
            "GB/s": 2 * nbytes / (ms * 1e-3) / 1e9}


# ------------------------------------------------------------------ traffic
TRAFFIC_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "prefill": ["plx_fwd.hip", "plx_common.hpp"],
    "decode": ["plx_decode.hip", "plx_common.hpp"],
    "decode_long": ["plx_decode.hip", "plx_common.hpp"],
    "decode_g16": ["plx_decode.hip", "plx_common.hpp"],
    "bwd": ["plx_bwd.hip", "plx_common.hpp"],
    "proj": ["plx_proj.hip", "plx_common.hpp"],
}


def source_digest(key):
    """Digest of the kernel sources with comments and whitespace removed, so
    that only a change to the code itself invalidates a counter summary."""
    import hashlib
    import re

    h = hashlib.sha256()
    for name in KERNEL_SOURCES[key]:
        with open(os.path.join(ROOT, "parallax_local_linear_plx_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(key):
    """HBM bytes per launch of the dominant kernel, from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE scaled by the copy calibration), or None
    when no summary exists or the kernel source changed since it was taken."""
    path = os.path.join(TRAFFIC_DIR, f"traffic_{key}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for ln in open(path):
        if ":" in ln:
            k, v = ln.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_digest") != source_digest(key):
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------- CPU baseline
def cpu_baseline(budget_s=12.0):
    """The fp64 oracle on sampled rows of the prefill workload, on host cores.
    Rate in the headline's unit (TFLOP/s over the four GEMM-equivalents)."""
    from oracle import plx_oracle as orc
    from parallax_local_linear_plx_amd import inputs

    T, d = 4096, 128
    wl = inputs.make_prefill(1, 2, 1, T, d, dtype="bf16", seed=2, rho_projected=True)
    ten = wl.tensors
    g = np.random.default_rng(0)
    flops = 0
    n_rows = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s or n_rows < 8:
        h = int(g.integers(2))
        i = int(g.integers(T))
        orc.row_forward(ten["q"].f64_slice((0, h, i)), ten["k"].f64_slice((0, 0, slice(0, i + 1))),
                        ten["v"].f64_slice((0, 0, slice(0, i + 1))), ten["rho"].f64_slice((0, h, i)),
                        wl.scale)
        flops += 4 * 2 * d * (i + 1)
        n_rows += 1
    dt = time.perf_counter() - t0
    blas, threads = "unknown", 1
    try:
        from threadpoolctl import threadpool_info

        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if pools:
            threads = max(p.get("num_threads", 1) for p in pools)
            blas = ", ".join(f"{p.get('internal_api')} {p.get('version')}" for p in pools)
    except Exception:  # pragma: no cover
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    cpu_model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                cpu_model = ln.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    # the oracle's cost per row is proportional to its key count i + 1, and
    # the rows were drawn uniformly, so the whole workload (B=4, Hq=16 rows
    # of every length 1..4096) scales linearly from the sample
    whole_units = 4 * 16 * T * (T + 1) // 2
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_rows} random rows (uniform i in [0,4096)) of the B=4 Hq=16 T=4096 d=128 "
                      f"prefill, fp64 numpy with explicit covariance per row, {dt:.1f} s",
            "affinity_cores": int(affinity), "cpu_model": cpu_model, "blas": blas,
            "seconds_sampled": round(dt, 2),
            "seconds_whole_workload_extrapolated": round(dt * whole_units / (flops / (8 * d)), 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU raises its clocks only after tens of milliseconds of sustained
    # work, so the default warm-up is long enough (>= ~40 ms per workload) to
    # time the steady state rather than the ramp.
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--only", default="all",
                    choices=["all", "prefill", "decode", "decode_long", "decode_g16", "train", "proj",
                             "copy", "decode_sweep", "headdim", "peaks"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay decode timing")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the operator shards by (batch, kv head) with no exchange, see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from parallax_local_linear_plx_amd import binding

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    binding.lib()  # fail loudly if the HIP library is missing

    res = {}
    if args.only in ("all", "prefill"):
        log("prefill ...")
        res["prefill"] = bench_prefill(args.steps, args.warmup)
        log(f"  {res['prefill']['ms'] * 1e3:.1f} us  {res['prefill']['tflops']:.1f} TFLOP/s")
    if args.only == "copy":
        print(json.dumps(bench_copy(args.steps)), flush=True)
        return
    if args.only == "peaks":
        print(json.dumps(measured_peaks()), flush=True)
        return
    if args.only == "headdim":
        log("head-dim variants ...")
        print(json.dumps({"metric": "prefill and backward TFLOP/s, decode GB/s at d = 64 and 256", "n_gpus": 1,
                          "dtype": "bf16", "data": "synthetic",
                          "headdim": bench_headdim(max(10, args.steps // 2), max(10, args.warmup // 2))}),
              flush=True)
        return
    if args.only == "decode_sweep":
        log("decode sweep (batch x context) ...")
        sweep = bench_decode_sweep(max(10, args.steps // 2), max(10, args.warmup // 3))
        print(json.dumps({"metric": "decode us/step and HBM GB/s over batch x context", "n_gpus": 1,
                          "higher_is_better": False, "unit": "us/step", "dtype": "bf16",
                          "data": "synthetic", "decode_sweep": sweep}), flush=True)
        return
    if args.only in ("all", "decode"):
        log("decode B64 ctx8192 ...")
        res["decode"] = bench_decode(args.steps, args.warmup, 64, [8192] * 64, 8192,
                                     "bf16 decode B=64 Hq=16 Hkv=8 ctx=8192 d=128", 31, not args.no_graph)
        log(f"  {res['decode']['us_per_step']:.1f} us  {res['decode']['GB/s']:.0f} GB/s")
    if args.only in ("all", "decode_long"):
        from parallax_local_linear_plx_amd import inputs

        ctx = inputs.long_decode_ctx()
        log(f"long decode B8 ctx {ctx.tolist()} ...")
        res["decode_long"] = bench_decode(args.steps, args.warmup, 8, ctx, 131072,
                                          "bf16 long-context decode B=8 Hq=16 Hkv=8 "
                                          "ctx~U{16384..131072} d=128, split-K", 41, not args.no_graph)
        log(f"  {res['decode_long']['us_per_step']:.1f} us  {res['decode_long']['GB/s']:.0f} GB/s")
    if args.only in ("all", "decode_g16"):
        # sixteen query heads per KV head: the kernel's two column groups share
        # one pass over the cache
        log("decode B64 Hq16 Hkv1 ctx8192 ...")
        res["decode_g16"] = bench_decode(args.steps, args.warmup, 64, [8192] * 64, 8192,
                                         "bf16 decode B=64 Hq=16 Hkv=1 (G=16) ctx=8192 d=128", 35,
                                         not args.no_graph, Hq=16, Hkv=1)
        log(f"  {res['decode_g16']['us_per_step']:.1f} us  {res['decode_g16']['GB/s']:.0f} GB/s")
    if args.only in ("all", "proj"):
        log("stacked projection ...")
        res["proj"] = bench_proj(args.steps, args.warmup)
        log(f"  {res['proj']['us_per_call']:.1f} us  {res['proj']['tflops']:.1f} TFLOP/s "
            f"(library matmul {res['proj']['library_matmul_us']:.1f} us)")
    if args.only in ("all", "train"):
        log("training step ...")
        res["train"] = bench_train(max(3, args.steps // 4), max(1, args.warmup // 2))
        log(f"  fwd {res['train']['fwd_ms']:.2f} ms  bwd {res['train']['bwd_ms']:.2f} ms")

    peaks = None
    if args.only == "all":
        log("measured ceilings ...")
        peaks = measured_peaks()
        log(f"  MFMA bf16 {peaks['mfma_bf16_tflops']:.0f} TFLOP/s, HBM read {peaks['hbm_read_gbs']:.0f} GB/s")

    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded device draws, q,k,v~N(0,1), rho=W_R x / N(0,0.1^2))"}
    if "prefill" in res:
        p = res["prefill"]
        line.update({"value": round(p["tflops"], 2), "unit": "TFLOP/s", "ms_per_step": round(p["ms"], 4),
                     "config": p["config"],
                     "roofline": {"bound": "mfma", "achieved": round(p["tflops"], 2),
                                  "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(p["tflops"] / PEAK_BF16_TFLOPS, 4),
                                  "traffic": measured_traffic("prefill"),
                                  "kernel": "fwd16_kernel<128,8,1,false>",
                                  **({"measured_peak": peaks["mfma_bf16_tflops"],
                                      "frac_of_measured": round(p["tflops"] / peaks["mfma_bf16_tflops"], 4)}
                                     if peaks else {}),
                                  "algorithmic_flops_per_launch": p["flops"]}})
    else:
        line.update({"value": None, "unit": "TFLOP/s", "ms_per_step": None, "config": {"workload": args.only}})
    for key in ("decode", "decode_long", "decode_g16", "train", "proj"):
        if key in res:
            line[key] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in res[key].items()}
            if key.startswith("decode"):
                r = res[key]
                line[key]["roofline"] = {
                    "bound": "hbm", "achieved": round(r["GB/s"], 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(r["GB/s"] / PEAK_HBM_GBS, 4),
                    "traffic": measured_traffic(key),
                    "kernel": (f"decode16_balanced_kernel<128,{16 if key == 'decode_g16' else 2}> + "
                               "decode_merge_balanced_kernel<128>"),
                    **({"measured_peak": peaks["hbm_read_gbs"],
                        "frac_of_measured": round(r["GB/s"] / peaks["hbm_read_gbs"], 4)} if peaks else {}),
                    "algorithmic_bytes_per_launch": r["bytes"]}
    if "train" in res:
        r = res["train"]
        line["train"]["roofline"] = {
            "bound": "mfma", "achieved": round(r["bwd_tflops"], 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(r["bwd_tflops"] / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic("bwd"), "kernel": "plx_bwd (all of its kernels)",
            "algorithmic_flops_per_launch": r["bwd_flops"]}
    line["clock_warmup_ms"] = CLOCK_WARM_MS
    if peaks:
        line["measured_peaks"] = peaks
    if not args.no_cpu and args.only in ("all", "prefill"):
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
