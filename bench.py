#!/usr/bin/env python3
"""Benchmark of the fused decode-MLP path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only gemv|all] [--cpu-seconds S]

A step is one call of the SwiGLU-prologue int4 GEMV at M=1, K=9216, N=2560 (the
single-row decode shape whose unfused form writes a 94 MB fp32 product), with its
fp32 output scale, over one of S rotating sets of seeded synthetic inputs already
resident in HBM.  The sets total more than twice the 256 MB Infinity Cache, so every
step streams its weights from HBM.  K steps are captured into hipGraphs (one per
rotation of the sets) and timed with HIP events on the stream they run on.

The JSON line on stdout reports achieved algorithmic GB/s (the job's bytes over the
time) and its fraction of MI355X's 8 TB/s HBM peak, the fp64 CPU oracle timed on this
host on a bounded sample, and, unless --only gemv, the other workloads: residual add +
RMSNorm at 8192 x 4096, the 16-row Llama-3-8B-sized MLP layer, a 16-row
Qwen2.5-1.5B-shaped layer, the 28-layer Qwen2.5-1.5B-sized MLP chain (eager and as one
hipGraph), the unfused sequences and a plain copy kernel.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/call + achieved HBM GB/s (% of peak), SwiGLU→W4 GEMV M=1 K=9216 N=2560"
PEAK_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 matrix peak
WORKLOAD = "swiglu_w4_gemv_1x9216x2560"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_swiglu_w4_gemv_1x9216x2560.json")
CALIB_FLOATS = 1 << 27          # calibration copy: 512 MiB read, 512 MiB written per launch (beyond every cache)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    from memory_bound_decode_add_amd.profiling import source_hash
    return source_hash()


def load_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; None otherwise."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


class Timer:
    """HIP events recorded on the current (launch) stream."""

    def __init__(self, torch):
        self.torch = torch

    def __call__(self, fn, reps=1):
        t = self.torch
        s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        t.cuda.synchronize()
        return s.elapsed_time(e) / 1e3     # seconds


def capture(torch, fns):
    """Capture a list of launch callables into one CUDA(HIP) graph."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for f in fns:
                f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


# ----------------------------------------------------------------------------
# the metric: SwiGLU-prologue W4 GEMV, M=1 K=9216 N=2560
# ----------------------------------------------------------------------------
def bench_gemv(torch, F, synth, steps, warmup, n_sets):
    from memory_bound_decode_add_amd import traffic as T
    c = synth.CONFIGS[WORKLOAD]
    M, K, N = c["M"], c["K"], c["N"]
    log(f"[bench] generating {n_sets} input sets for M={M} K={K} N={N}")
    sets = []
    for i in range(n_sets):
        inp = synth.swiglu_gemv_inputs(M, K, N, seed=i, out_scale=c["out_scale"])
        sets.append((F.from_bits(inp.g), F.from_bits(inp.u), F.W4Weight.from_numpy(inp.W.qweight, inp.W.scales),
                     torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))
    scale = F.scalar(c["out_scale"])
    ws = F.workspace(F.gemv_workspace_bytes(M, K, N))
    bytes_per_call = T.swiglu_w4_gemv_bytes(M, K, N)

    def step(i):
        g, u, W, y = sets[i % n_sets]
        return lambda: F.swiglu_w4_gemv(g, u, W, scale, None, out=y, ws=ws)

    # One graph of a full rotation (every set once, in order) and one of the first
    # `steps mod n_sets` sets.  The timed region is floor(steps / n_sets) full rotations and
    # then the remainder, right after a full rotation: whatever `steps` is, a timed call's
    # set was last read n_sets calls earlier, with n_sets * bytes_per_call (more than twice
    # the Infinity Cache) read in between.
    g_full = capture(torch, [step(i) for i in range(n_sets)])
    rem = steps % n_sets
    g_rem = capture(torch, [step(i) for i in range(rem)]) if rem else None
    done = 0
    while done < max(warmup, n_sets):
        g_full.replay()
        done += n_sets
    if g_rem is not None:                  # upload it, then a full rotation again
        g_rem.replay()
        g_full.replay()
        done += rem + n_sets
    torch.cuda.synchronize()

    timer = Timer(torch)

    def timed():
        for _ in range(steps // n_sets):
            g_full.replay()
        if g_rem is not None:
            g_rem.replay()

    elapsed = timer(timed)
    us = elapsed / steps * 1e6
    gbps = bytes_per_call / (elapsed / steps) / 1e9

    # the spread: 20 separately timed rotations, each followed by an untimed 12 MB copy (so
    # that clock and cache drift hit every round alike)
    cpy_src = torch.randn(int(12.2e6 / 8), device="cuda")
    cpy_dst = torch.empty_like(cpy_src)
    rounds = []
    for _ in range(20):
        rounds.append(timer(g_full.replay) / n_sets * 1e6)
        torch.neg(cpy_src, out=cpy_dst)
    torch.cuda.synchronize()
    del cpy_src, cpy_dst
    spread = {"rounds": len(rounds), "calls_per_round": n_sets, "median_us": float(np.median(rounds)),
              "p10_us": float(np.percentile(rounds, 10)), "p90_us": float(np.percentile(rounds, 90))}

    ceiling = measured_ceiling(torch, F, timer, sets, n_sets, K, N)
    ceiling["gemv_frac_of_read_only"] = ceiling["read_only_us"] / us
    ceiling["gemv_us_above_floor"] = us - ceiling["empty_kernel_us"]
    ceiling["read_only_us_above_floor"] = ceiling["read_only_us"] - ceiling["empty_kernel_us"]

    # a plain copy kernel of known size, for scaling the HBM byte counters of a profiled run
    src = torch.randn(CALIB_FLOATS, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(8):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst

    # single eagerly launched call (launch latency included), median of 20
    lat = []
    g, u, W, y = sets[0]
    for _ in range(20):
        lat.append(timer(lambda: F.swiglu_w4_gemv(g, u, W, scale, None, out=y, ws=ws)))
    plan = {"workspace_bytes": F.gemv_workspace_bytes(M, K, N)}
    timed_sets = min(steps, n_sets)
    return {"us_per_call": us, "gbps": gbps, "elapsed_s": elapsed, "bytes_per_call": bytes_per_call,
            "warmup_steps_run": done, "timed_steps": steps, "rotating_input_sets": n_sets,
            "distinct_sets_timed": timed_sets, "bytes_read_between_reuses_of_a_set": n_sets * bytes_per_call,
            "eager_call_us_median": float(np.median(lat)) * 1e6, "rounds": spread, "measured_ceiling": ceiling,
            **plan}


def measured_ceiling(torch, F, timer, sets, n_sets, K, N):
    """The per-call floor and ceiling the GEMV is measured against, timed like it (one
    graph of n_sets back-to-back launches, replayed): an empty kernel on the GEMV's grid,
    and a kernel that only reads the GEMV's bytes in the column kernel's order (its
    workgroup's columns' packed weights, all of g and u, its columns' group scales) over
    the same rotating sets, writing one word per workgroup."""
    wgs = 256
    cols = N // wgs
    per_wg = cols * (K // 32)                 # 16-byte chunks of the workgroup's columns
    sink = torch.empty(wgs, dtype=torch.int32, device="cuda")
    g_empty = capture(torch, [lambda: F.empty_kernel(wgs, 1024) for _ in range(n_sets)])
    g_read = capture(torch, [lambda s=s: F.read_ceiling(s[2].qweight, per_wg, s[0], s[1], s[2].scales, K // 128,
                                                        2 * N, 2 * cols, wgs, sink) for s in sets])
    for g in (g_empty, g_read, g_read):
        g.replay()
    torch.cuda.synchronize()
    reps = 10
    t_empty = timer(g_empty.replay, reps) / (reps * n_sets)
    t_read = timer(g_read.replay, reps) / (reps * n_sets)
    del g_empty, g_read
    return {"empty_kernel_us": t_empty * 1e6, "read_only_us": t_read * 1e6,
            "read_only_bytes": K * N // 2 + 2 * K * 2 + (K // 128) * 2 * N,
            "timing": f"graph of {n_sets} back-to-back launches over the rotating sets, {reps} replays"}


def bench_repeat(torch, timer, fns, n_rep):
    """Time n_rep replays of a graph of the given launches; seconds per launch list."""
    g = capture(torch, fns)
    g.replay()
    torch.cuda.synchronize()
    return timer(g.replay, n_rep) / n_rep


def bench_extras(torch, F, synth, n_sets_gemv):
    from memory_bound_decode_add_amd import traffic as T
    timer = Timer(torch)
    out = {}

    # a plain copy kernel (torch's elementwise negation: n*4 bytes in, n*4 out), size-matched
    # to the GEMV's and the norm's traffic, rotating over >= 600 MB of buffers
    for mb in (12.2, 268.4):
        n = int(mb * 1e6 / 8)
        sets = [(torch.randn(n, device="cuda"), torch.empty(n, device="cuda")) for _ in range(max(2, int(600 / mb)))]
        t = bench_repeat(torch, timer, [lambda s=s: torch.neg(s[0], out=s[1]) for s in sets], 5) / len(sets)
        out[f"copy_{mb}MB_total"] = {"us": t * 1e6, "gbps_rw": 2 * n * 4 / t / 1e9}
        del sets

    # residual add + RMSNorm, 8192 x 4096, 4 rotating sets (1.07 GB)
    c = synth.CONFIGS["add_rmsnorm_8192x4096"]
    M, H = c["M"], c["H"]
    log("[bench] add_rmsnorm 8192x4096")
    sets = []
    for i in range(4):
        inp = synth.add_rmsnorm_inputs(M, H, seed=i)
        sets.append((F.from_bits(inp.x), F.from_bits(inp.r), F.from_bits(inp.w),
                     torch.empty((M, H), dtype=torch.bfloat16, device="cuda"),
                     torch.empty((M, H), dtype=torch.bfloat16, device="cuda")))
    fns = [lambda s=s: F.add_rmsnorm(s[0], s[1], s[2], c["eps"], h_out=s[3], y_out=s[4]) for s in sets]
    t = bench_repeat(torch, timer, fns, 10) / len(sets)
    b = T.add_rmsnorm_bytes(M, H)
    out["add_rmsnorm_8192x4096"] = {"us_per_call": t * 1e6, "gbps": b / t / 1e9, "frac_of_peak": b / t / 1e9 / PEAK_GBPS}
    wsn = F.workspace(F.unfused_add_rmsnorm_workspace_bytes(M, H))
    fns = [lambda s=s: F.unfused_add_rmsnorm(s[0], s[1], s[2], c["eps"], h_out=s[3], y_out=s[4], ws=wsn)
           for s in sets[:2]]
    t = bench_repeat(torch, timer, fns, 4) / 2
    out["unfused_add_rmsnorm_8192x4096"] = {"us_per_call": t * 1e6, "kernels": 9,
                                            "gbps_actual_bytes": T.add_rmsnorm_eager_bytes(M, H) / t / 1e9}
    del sets, wsn

    # unfused sequences at the metric shape
    c = synth.CONFIGS[WORKLOAD]
    Mg, K, N = c["M"], c["K"], c["N"]
    log("[bench] unfused GEMV sequences")
    gsets = []
    for i in range(min(n_sets_gemv, 48)):
        inp = synth.swiglu_gemv_inputs(Mg, K, N, seed=i, out_scale=c["out_scale"])
        gsets.append((F.from_bits(inp.g), F.from_bits(inp.u), F.W4Weight.from_numpy(inp.W.qweight, inp.W.scales),
                      torch.empty((Mg, N), dtype=torch.bfloat16, device="cuda")))
    scale = F.scalar(c["out_scale"])
    for mode, name in ((F.UNFUSED_PRODUCT, "product"), (F.UNFUSED_ACT, "act")):
        wsu = F.workspace(F.unfused_gemv_workspace_bytes(mode, Mg, K, N))
        fns = [lambda s=s, wsu=wsu, mode=mode: F.unfused_swiglu_w4_gemv(mode, s[0], s[1], s[2], scale, out=s[3],
                                                                          ws=wsu) for s in gsets]
        t = bench_repeat(torch, timer, fns, 2) / len(gsets)
        ab = T.unfused_product_gemv_bytes(K, N) if mode == F.UNFUSED_PRODUCT else T.unfused_act_gemv_bytes(Mg, K, N)
        out[f"unfused_{name}_1x9216x2560"] = {"us_per_call": t * 1e6, "gbps_actual_bytes": ab / t / 1e9,
                                              "workspace_bytes": F.unfused_gemv_workspace_bytes(mode, Mg, K, N)}
        del wsu

    # batch sweep at the metric's K and N: the same 48 rotating weight sets, M rows of
    # seeded N(0,1) activations, one graph per batch size; M <= 4 runs the column kernel,
    # 5 <= M <= 16 the matrix-core kernel, M = 32 and 64 the same kernel with two and four
    # 16-row blocks per weight load
    log("[bench] batch sweep M=1..64 at K=9216 N=2560")
    gen = torch.Generator().manual_seed(1234)
    sweep = {}
    for Mb in (1, 2, 3, 4, 5, 8, 12, 16, 32, 64):
        gb = torch.randn(Mb, K, generator=gen).to(torch.bfloat16).cuda()
        ub = torch.randn(Mb, K, generator=gen).to(torch.bfloat16).cuda()
        ys = [torch.empty((Mb, N), dtype=torch.bfloat16, device="cuda") for _ in gsets]
        wsb = F.workspace(F.gemv_workspace_bytes(Mb, K, N))
        fns = [lambda s=s, y=y: F.swiglu_w4_gemv(gb, ub, s[2], scale, out=y, ws=wsb) for s, y in zip(gsets, ys)]
        t = bench_repeat(torch, timer, fns, 5) / len(gsets)
        b = T.swiglu_w4_gemv_bytes(Mb, K, N)
        sweep[f"M{Mb}"] = {"us_per_call": t * 1e6, "gbps": b / t / 1e9, "frac_of_peak": b / t / 1e9 / PEAK_GBPS,
                           "kernel": F.gemv_kernel(Mb, K, N)}
        del gb, ub, ys, wsb
    out["batch_sweep_swiglu_w4_gemv_9216x2560"] = sweep
    del gsets

    # the same SwiGLU GEMV with FP4 weights (E2M1 + E4M3 1x16 block scales), 48
    # rotating sets (13.3 MB each, 639 MB in all)
    log("[bench] FP4 SwiGLU GEMV M=1 K=9216 N=2560")
    fsets = []
    for i in range(min(n_sets_gemv, 48)):
        inp = synth.swiglu_fp4_gemv_inputs(Mg, K, N, seed=i, out_scale=c["out_scale"])
        fsets.append((F.from_bits(inp.g), F.from_bits(inp.u), F.FP4Weight.from_numpy(inp.W.qweight, inp.W.scales),
                      torch.empty((Mg, N), dtype=torch.bfloat16, device="cuda")))
    fns = [lambda s=s: F.swiglu_fp4_gemv(s[0], s[1], s[2], scale, out=s[3]) for s in fsets]
    t = bench_repeat(torch, timer, fns, 5) / len(fsets)
    b = T.swiglu_fp4_gemv_bytes(Mg, K, N)
    out["swiglu_fp4_gemv_1x9216x2560"] = {"us_per_call": t * 1e6, "gbps": b / t / 1e9,
                                          "frac_of_peak": b / t / 1e9 / PEAK_GBPS, "bytes_per_call": b}
    # the same weights at 16 and 64 rows (the matrix-core kernel with FP4 weights; 64 rows
    # as four 16-row blocks per weight load)
    gen = torch.Generator().manual_seed(4321)
    for Mb in (16, 64):
        gb = torch.randn(Mb, K, generator=gen).to(torch.bfloat16).cuda()
        ub = torch.randn(Mb, K, generator=gen).to(torch.bfloat16).cuda()
        ys = [torch.empty((Mb, N), dtype=torch.bfloat16, device="cuda") for _ in fsets]
        wsb = F.workspace(F.fp4_gemv_workspace_bytes(Mb, K, N))
        fns = [lambda s=s, y=y: F.swiglu_fp4_gemv(gb, ub, s[2], scale, out=y, ws=wsb) for s, y in zip(fsets, ys)]
        t = bench_repeat(torch, timer, fns, 5) / len(fsets)
        b = T.swiglu_fp4_gemv_bytes(Mb, K, N)
        out[f"swiglu_fp4_gemv_{Mb}x9216x2560"] = {"us_per_call": t * 1e6, "gbps": b / t / 1e9,
                                                  "frac_of_peak": b / t / 1e9 / PEAK_GBPS, "bytes_per_call": b}
        del gb, ub, ys, wsb

    # both operands FP4: the SwiGLU activation quantised to E2M1 with E4M3 1x16 block scales
    # in the prologue, over a per-tensor scale calibrated once from one set's activation
    # (largest magnitude / (6 * 448)); the HBM bytes are those of the FP4-weight GEMV
    log("[bench] FP4-activation SwiGLU GEMV 1/16/64 x 9216x2560")
    gen = torch.Generator().manual_seed(4444)
    for Mb in (1, 16, 64):
        gb = torch.randn(Mb, K, generator=gen).to(torch.bfloat16).cuda()
        ub = torch.randn(Mb, K, generator=gen).to(torch.bfloat16).cuda()
        gsc = F.scalar(F.swiglu(gb, ub).float().abs().max().item() / (6.0 * 448.0))
        ys = [torch.empty((Mb, N), dtype=torch.bfloat16, device="cuda") for _ in fsets]
        wsb = F.workspace(max(1, F.fp4_gemv_workspace_bytes(Mb, K, N)))
        fns = [lambda s=s, y=y: F.swiglu_fp4a4_gemv(gb, ub, s[2], gsc, scale, out=y, ws=wsb)
               for s, y in zip(fsets, ys)]
        t = bench_repeat(torch, timer, fns, 5) / len(fsets)
        b = T.swiglu_fp4_gemv_bytes(Mb, K, N)
        out[f"swiglu_fp4a4_gemv_{Mb}x9216x2560"] = {"us_per_call": t * 1e6, "gbps": b / t / 1e9,
                                                    "frac_of_peak": b / t / 1e9 / PEAK_GBPS, "bytes_per_call": b}
        del gb, ub, ys, wsb
    del fsets

    # the prefill point: 2,048 tokens through the SwiGLU pass and the matrix-core GEMM at
    # the metric's K and N (4 rotating weight sets; the activation is 75 MB per call anyway)
    log("[bench] prefill 2048x9216x2560")
    Mp = 2048
    psets = [F.W4Weight.from_numpy(*(lambda w: (w.qweight, w.scales))(
        synth.swiglu_gemv_inputs(1, K, N, seed=100 + i).W)) for i in range(4)]
    gen = torch.Generator().manual_seed(2048)
    gp = torch.randn(Mp, K, generator=gen).to(torch.bfloat16).cuda()
    up = torch.randn(Mp, K, generator=gen).to(torch.bfloat16).cuda()
    actp = torch.empty((Mp, K), dtype=torch.bfloat16, device="cuda")
    yps = [torch.empty((Mp, N), dtype=torch.bfloat16, device="cuda") for _ in psets]
    wsp = F.workspace(F.swiglu_w4_gemm_workspace_bytes(Mp, K))
    t_act = bench_repeat(torch, timer, [lambda: F.swiglu(gp, up, out=actp)], 10)
    t_gemm = bench_repeat(torch, timer, [lambda W=W, y=y: F.w4_gemm(actp, W, scale, out=y) for W, y in zip(psets, yps)],
                          5) / len(psets)
    t_all = bench_repeat(torch, timer, [lambda W=W, y=y: F.swiglu_w4_gemm(gp, up, W, scale, out=y, ws=wsp)
                                        for W, y in zip(psets, yps)], 5) / len(psets)
    flops = 2.0 * Mp * K * N
    out["prefill_swiglu_w4_gemm_2048x9216x2560"] = {
        "us_per_call": t_all * 1e6, "swiglu_pass_us": t_act * 1e6, "gemm_us": t_gemm * 1e6,
        "swiglu_pass_gbps": 3 * Mp * K * 2 / t_act / 1e9,
        "gemm_roofline": {"bound": "mfma", "achieved": flops / t_gemm / 1e12, "peak": PEAK_BF16_TFLOPS,
                          "unit": "TFLOP/s", "frac": flops / t_gemm / 1e12 / PEAK_BF16_TFLOPS},
        "kernels": 2}
    del psets, gp, up, actp, yps, wsp

    # Llama-3-8B-sized MLP layer at M=16, 6 rotating weight sets
    c = synth.CONFIGS["mlp_llama3_8b_m16"]
    M, H, I = c["M"], c["H"], c["I"]
    log("[bench] MLP layer M=16 H=4096 I=14336")
    layers = []
    for i in range(6):
        inp = synth.mlp_inputs(M, H, I, 1, seed=i, out_scale=c["out_scale"])
        L = inp.layers[0]
        layers.append(F.MlpLayer(F.from_bits(L.norm_w), F.W4Weight.from_numpy(L.gate_up.qweight, L.gate_up.scales),
                                 F.W4Weight.from_numpy(L.down.qweight, L.down.scales), F.scalar(L.out_scale),
                                 L.eps, True))
    bufs = F.MlpBuffers.empty(M, H, I)
    bufs.x.copy_(F.from_bits(inp.x))
    bufs.residual.copy_(F.from_bits(inp.r))
    wsm = F.workspace(F.mlp_workspace_bytes(M, H, I))
    t = bench_repeat(torch, timer, [lambda L=L: F.mlp_decode(L, bufs, wsm) for L in layers], 5) / len(layers)
    b = T.mlp_layer_bytes(M, H, I, True)
    out["mlp_llama3_8b_m16"] = {"us_per_call": t * 1e6, "gbps": b / t / 1e9, "frac_of_peak": b / t / 1e9 / PEAK_GBPS}
    wsu = F.workspace(F.unfused_mlp_workspace_bytes(M, H, I))
    t = bench_repeat(torch, timer, [lambda L=L: F.unfused_mlp_decode(L, bufs, wsu) for L in layers[:2]], 3) / 2
    out["unfused_mlp_llama3_8b_m16"] = {"us_per_call": t * 1e6}
    # the same layer with SwiGLU as the gate_up epilogue (norm; gate_up + SwiGLU writing act
    # [16, I]; down with the residual), and its gate_up kernel alone
    b2 = F.Mlp2Buffers.empty(M, H, I)
    b2.x.copy_(bufs.x)
    b2.residual.copy_(bufs.residual)
    ws2 = F.workspace(F.mlp2_workspace_bytes(M, H, I))
    t = bench_repeat(torch, timer, [lambda L=L: F.mlp_decode2(L, b2, ws2) for L in layers], 5) / len(layers)
    b = T.mlp2_layer_bytes(M, H, I, True)
    out["mlp2_llama3_8b_m16"] = {"us_per_call": t * 1e6, "gbps": b / t / 1e9, "frac_of_peak": b / t / 1e9 / PEAK_GBPS,
                                 "bytes_per_call": b, "kernels": 3}
    yb = torch.empty((M, H), dtype=torch.bfloat16, device="cuda").normal_()
    wsp = F.workspace(F.w4_gemv_swiglu_workspace_bytes(M, H, I))
    t = bench_repeat(torch, timer, [lambda L=L: F.w4_gemv_swiglu(yb, L.gate_up, out=b2.act, ws=wsp)
                                    for L in layers], 5) / len(layers)
    b = T.w4_gemv_swiglu_bytes(M, H, I)
    out["w4_gemv_swiglu_16x4096x14336"] = {"us_per_call": t * 1e6, "gbps": b / t / 1e9,
                                            "frac_of_peak": b / t / 1e9 / PEAK_GBPS, "bytes_per_call": b}
    del layers, bufs, wsm, wsu, b2, ws2, yb, wsp

    # one Qwen2.5-1.5B-shaped layer at 16 rows (H=1536, I=8960: short K, where the GEMVs run
    # on the kernel fed by direct-to-LDS loads), both layer forms, 6 rotating weight sets
    M16, H16, I16 = 16, 1536, 8960
    log(f"[bench] MLP layer M={M16} H={H16} I={I16}")
    layers = []
    for i in range(6):
        L = synth.mlp_inputs(M16, H16, I16, 1, seed=50 + i, out_scale=1.0).layers[0]
        layers.append(F.MlpLayer(F.from_bits(L.norm_w), F.W4Weight.from_numpy(L.gate_up.qweight, L.gate_up.scales),
                                 F.W4Weight.from_numpy(L.down.qweight, L.down.scales), F.scalar(L.out_scale),
                                 L.eps, True))
    gen = torch.Generator().manual_seed(16)
    xq = torch.randn(M16, H16, generator=gen).to(torch.bfloat16).cuda()
    bufs = F.MlpBuffers.empty(M16, H16, I16)
    bufs.x.copy_(xq)
    bufs.residual.copy_(xq)
    wsm = F.workspace(F.mlp_workspace_bytes(M16, H16, I16))
    t = bench_repeat(torch, timer, [lambda L=L: F.mlp_decode(L, bufs, wsm) for L in layers], 10) / len(layers)
    b = T.mlp_layer_bytes(M16, H16, I16, True)
    out["mlp_qwen2_5_1_5b_m16"] = {"us_per_call": t * 1e6, "gbps": b / t / 1e9, "frac_of_peak": b / t / 1e9 / PEAK_GBPS}
    b2 = F.Mlp2Buffers.empty(M16, H16, I16)
    b2.x.copy_(xq)
    b2.residual.copy_(xq)
    ws2 = F.workspace(F.mlp2_workspace_bytes(M16, H16, I16))
    t = bench_repeat(torch, timer, [lambda L=L: F.mlp_decode2(L, b2, ws2) for L in layers], 10) / len(layers)
    b = T.mlp2_layer_bytes(M16, H16, I16, True)
    out["mlp2_qwen2_5_1_5b_m16"] = {"us_per_call": t * 1e6, "gbps": b / t / 1e9, "frac_of_peak": b / t / 1e9 / PEAK_GBPS}
    del layers, bufs, wsm, b2, ws2, xq

    # Qwen2.5-1.5B-sized MLP chain, 28 layers: eager chain vs one hipGraph
    c = synth.CONFIGS["mlp_qwen2_5_1_5b_28l"]
    M, H, I, NL = c["M"], c["H"], c["I"], c["n_layers"]
    log("[bench] 28-layer MLP chain M=1 H=1536 I=8960")
    inp = synth.mlp_inputs(M, H, I, NL, seed=0, out_scale=c["out_scale"])
    layers = [F.MlpLayer(F.from_bits(L.norm_w), F.W4Weight.from_numpy(L.gate_up.qweight, L.gate_up.scales),
                         F.W4Weight.from_numpy(L.down.qweight, L.down.scales), F.scalar(L.out_scale), L.eps, False)
              for L in inp.layers]
    bufs = F.MlpBuffers.empty(M, H, I, out_is_x=True)
    x0, r0 = F.from_bits(inp.x), F.from_bits(inp.r)
    wsc = F.workspace(F.mlp_workspace_bytes(M, H, I))
    graph = F.MlpGraph(layers, bufs, wsc)
    b = NL * T.mlp_layer_bytes(M, H, I, False)

    def reset():
        bufs.x.copy_(x0)
        bufs.residual.copy_(r0)

    reset()
    graph.launch()
    torch.cuda.synchronize()
    tg = timer(graph.launch, 20) / 20
    reset()
    F.mlp_chain(layers, bufs, wsc)
    torch.cuda.synchronize()
    te = timer(lambda: F.mlp_chain(layers, bufs, wsc), 20) / 20
    out["mlp_chain_qwen2_5_1_5b_28l"] = {"graph_us_per_step": tg * 1e6, "eager_us_per_step": te * 1e6,
                                         "kernels_per_step": graph.kernel_count, "bytes_per_step": b,
                                         "graph_gbps": b / tg / 1e9, "graph_frac_of_peak": b / tg / 1e9 / PEAK_GBPS}
    graph.close()

    # the same chain with the two-kernel layer (norm as the gate_up prologue, SwiGLU as
    # its epilogue)
    log("[bench] 28-layer two-kernel MLP chain M=1 H=1536 I=8960")
    bufs2 = F.Mlp2Buffers.empty(M, H, I, out_is_x=True)
    ws2 = F.workspace(F.mlp2_workspace_bytes(M, H, I))
    graph2 = F.Mlp2Graph(layers, bufs2, ws2)
    b2 = NL * T.mlp2_layer_bytes(M, H, I, False)

    def reset2():
        bufs2.x.copy_(x0)
        bufs2.residual.copy_(r0)

    reset2()
    graph2.launch()
    torch.cuda.synchronize()
    tg2 = timer(graph2.launch, 20) / 20
    reset2()
    F.mlp_chain2(layers, bufs2, ws2)
    torch.cuda.synchronize()
    te2 = timer(lambda: F.mlp_chain2(layers, bufs2, ws2), 20) / 20
    out["mlp2_chain_qwen2_5_1_5b_28l"] = {"graph_us_per_step": tg2 * 1e6, "eager_us_per_step": te2 * 1e6,
                                          "kernels_per_step": graph2.kernel_count, "bytes_per_step": b2,
                                          "graph_gbps": b2 / tg2 / 1e9,
                                          "graph_frac_of_peak": b2 / tg2 / 1e9 / PEAK_GBPS}

    # re-pointing the captured graph at a second set of buffers (same shapes): the
    # in-place parameter update against a fresh capture + instantiation, host time
    bufs2b = F.Mlp2Buffers.empty(M, H, I, out_is_x=True)
    ws2b = F.workspace(F.mlp2_workspace_bytes(M, H, I))
    cap = torch.cuda.Stream()
    t_upd, t_new = [], []
    for i in range(6):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph2.update(layers, bufs2b if i % 2 == 0 else bufs2, ws2b if i % 2 == 0 else ws2, stream=cap)
        t_upd.append(time.perf_counter() - t0)
        t0 = time.perf_counter()
        gfresh = F.Mlp2Graph(layers, bufs2b, ws2b, stream=cap)
        t_new.append(time.perf_counter() - t0)
        gfresh.close()
    bufs2.x.copy_(x0)
    bufs2.residual.copy_(r0)
    graph2.launch()
    torch.cuda.synchronize()
    tg2u = timer(graph2.launch, 20) / 20
    out["mlp2_chain_qwen2_5_1_5b_28l"].update({
        "graph_update_ms_median": float(np.median(t_upd)) * 1e3,
        "graph_create_ms_median": float(np.median(t_new)) * 1e3,
        "graph_us_per_step_after_update": tg2u * 1e6})
    graph2.close()
    return out


def host_info():
    """The host the CPU baseline runs on: core counts, affinity, CPU model, BLAS."""
    info = {"os_cpu_count": os.cpu_count()}
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        info["affinity_cpus"] = None
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    info["cpu_model"] = model
    blas_threads, blas_lib = 1, None
    try:
        from threadpoolctl import threadpool_info
        for d in threadpool_info():
            if d.get("user_api") == "blas":
                blas_threads = max(blas_threads, int(d.get("num_threads", 1)))
                blas_lib = f"{d.get('internal_api')} {d.get('version')} ({os.path.basename(d.get('filepath', ''))})"
    except Exception:
        pass
    info["blas"] = blas_lib
    info["blas_threads"] = blas_threads
    return info


def cpu_baseline(synth, seconds):
    """The fp64 oracle on the metric's workload, repeated for about `seconds` of CPU time."""
    import oracle as O
    from memory_bound_decode_add_amd import traffic as T
    host = host_info()
    blas = host["blas_threads"]
    c = synth.CONFIGS[WORKLOAD]
    inp = synth.swiglu_gemv_inputs(c["M"], c["K"], c["N"], seed=0, out_scale=c["out_scale"])
    n = 0
    t0 = time.perf_counter()
    while True:
        O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, c["out_scale"])
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 1000:
            break
    b = T.swiglu_w4_gemv_bytes(c["M"], c["K"], c["N"])
    return {"value": b * n / el / 1e9, "unit": "GB/s", "cores": int(blas), "kind": "oracle",
            "us_per_call": el / n * 1e6, "host": host,
            "sample": f"{n} oracle calls on input set 0 of {WORKLOAD} ({el:.1f} s, numpy fp64; elementwise on 1 "
                      f"thread, the fp64 matmul on {blas} BLAS threads)"}


def profile_calls(torch, F, synth):
    """A few eager calls of each kernel family, for hardware-counter runs:
    - the column kernel at the metric's shape (M=1, K=9216, N=2560, SwiGLU);
    - the matrix-core kernels at 16 rows: the kernel whose waves split K (K=9216, N=2560,
      SwiGLU), the row-block kernel on the Llama-3-8B-sized gate_up (K=4096, N=28672,
      identity) and the ring kernel on its down projection (K=14336, N=4096, SwiGLU, with
      its finish kernel) and on the Qwen2.5-1.5B-sized gate_up (K=1536, N=17920, identity);
    - the gate_up projection with the SwiGLU epilogue (M=16, K=4096, I=14336, pair mode);
    - the FP4 kernels at M=1 and 16 (K=9216, N=2560), with FP4 weights and with both
      operands FP4;
    - the prefill point: the SwiGLU pass and the W4 GEMM at 2048 x 9216 x 2560."""
    sc = F.scalar(0.5)
    for M, K, N, pro, n in ((1, 9216, 2560, "swiglu", 24), (16, 9216, 2560, "swiglu", 24),
                            (16, 4096, 28672, "id", 4), (16, 14336, 4096, "swiglu", 4), (16, 1536, 17920, "id", 8)):
        sets = []
        for i in range(n):
            inp = synth.swiglu_gemv_inputs(M, K, N, seed=i)
            sets.append((F.from_bits(inp.g), F.from_bits(inp.u), F.W4Weight.from_numpy(inp.W.qweight, inp.W.scales),
                         torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))
        ws = F.workspace(F.gemv_workspace_bytes(M, K, N))
        for _ in range(2):
            for g, u, W, y in sets:
                if pro == "swiglu":
                    F.swiglu_w4_gemv(g, u, W, sc, out=y, ws=ws)
                else:
                    F.w4_gemv(g, W, sc, out=y, ws=ws)
        torch.cuda.synchronize()
        del sets, ws
    M, K, I = 16, 4096, 14336
    sets = []
    for i in range(4):
        inp = synth.swiglu_gemv_inputs(M, K, 2 * I, seed=i)
        sets.append((F.from_bits(inp.g), F.W4Weight.from_numpy(inp.W.qweight, inp.W.scales),
                     torch.empty((M, I), dtype=torch.bfloat16, device="cuda")))
    ws = F.workspace(F.w4_gemv_swiglu_workspace_bytes(M, K, I))
    for _ in range(2):
        for x, W, act in sets:
            F.w4_gemv_swiglu(x, W, out=act, ws=ws)
    torch.cuda.synchronize()
    del sets, ws
    for M in (1, 16):
        inp = synth.swiglu_fp4_gemv_inputs(M, 9216, 2560, seed=M)
        g, u = F.from_bits(inp.g), F.from_bits(inp.u)
        W = F.FP4Weight.from_numpy(inp.W.qweight, inp.W.scales)
        y = torch.empty((M, 2560), dtype=torch.bfloat16, device="cuda")
        ws = F.workspace(F.fp4_gemv_workspace_bytes(M, 9216, 2560))
        gsc = F.scalar(F.swiglu(g, u).float().abs().max().item() / (6.0 * 448.0))
        for _ in range(8):
            F.swiglu_fp4_gemv(g, u, W, sc, out=y, ws=ws)
        for _ in range(8):
            F.swiglu_fp4a4_gemv(g, u, W, gsc, sc, out=y, ws=ws)
    torch.cuda.synchronize()
    M, K, N = 2048, 9216, 2560
    inp = synth.swiglu_gemv_inputs(1, K, N, seed=0)
    W = F.W4Weight.from_numpy(inp.W.qweight, inp.W.scales)
    gen = torch.Generator().manual_seed(2048)
    g = torch.randn(M, K, generator=gen).to(torch.bfloat16).cuda()
    u = torch.randn(M, K, generator=gen).to(torch.bfloat16).cuda()
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = F.workspace(F.swiglu_w4_gemm_workspace_bytes(M, K))
    for _ in range(4):
        F.swiglu_w4_gemm(g, u, W, F.scalar(1.0), out=y, ws=ws)
    torch.cuda.synchronize()
    log("[bench] profile calls done")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=480)
    ap.add_argument("--warmup", type=int, default=48)
    ap.add_argument("--sets", type=int, default=48, help="rotating input sets (48 x 12.2 MB = 586 MB)")
    ap.add_argument("--only", choices=["gemv", "all", "profile"], default="all",
                    help="profile: a few calls of each GEMV kernel family and exit (for counter runs)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if a.steps < 1:
        sys.exit("--steps must be >= 1")
    if a.sets < 2:
        sys.exit("--sets must be >= 2")

    import torch
    import memory_bound_decode_add_amd as F
    import synth
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    F.lib()   # fail loudly if the HIP library is missing
    if a.only == "profile":
        profile_calls(torch, F, synth)
        return

    res = bench_gemv(torch, F, synth, a.steps, a.warmup, a.sets)
    log(f"[bench] gemv: {res['us_per_call']:.3f} us/call, {res['gbps']:.1f} GB/s")
    extras = bench_extras(torch, F, synth, a.sets) if a.only == "all" else {}
    if extras:
        extras[f"measured_ceiling_{WORKLOAD}"] = res["measured_ceiling"]
    cpu = cpu_baseline(synth, a.cpu_seconds) if a.only == "all" and a.cpu_seconds > 0 else None

    traffic = load_traffic()
    line = {
        "metric": METRIC,
        "value": round(res["gbps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": res["us_per_call"] / 1e3,
        "us_per_call": round(res["us_per_call"], 4),
        "frac_of_peak": round(res["gbps"] / PEAK_GBPS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16*i4->f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "M": 1, "K": 9216, "N": 2560, "out_scale": 1.0,
                   "rotating_input_sets": a.sets, "distinct_sets_timed": res["distinct_sets_timed"],
                   "bytes_read_between_reuses_of_a_set": res["bytes_read_between_reuses_of_a_set"],
                   "bytes_per_call": res["bytes_per_call"],
                   "timing": "hipGraph replays of back-to-back calls after a full rotation of the sets, "
                             "HIP events on the launch stream"},
        "roofline": {"bound": "hbm", "achieved": round(res["gbps"], 2), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(res["gbps"] / PEAK_GBPS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "detail": {k: v for k, v in res.items() if k not in ("gbps",)},
        "extras": extras,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
