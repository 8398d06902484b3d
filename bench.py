#!/usr/bin/env python3
"""Benchmark of the RG-LRU temporal branch (conv width 4 -> RG-LRU) on one MI355X.

Headline workload: the training-shape forward B=8, T=2048, D_RNN=2560, bf16 I/O with
fp32 scan state.  One step is one call of the product entry point rglru_fwd over one batch:
its conv launch (K0, width-4 causal conv, which also initialises the look-back status) and
the fused RG-LRU kernel (K1: MFMA gate GEMM with the log-space gates and the chunked scan
in its epilogue).  Inputs are resident in HBM before the timed region; three input sets
rotate so consecutive steps do not re-read the same x from the 256 MB Infinity Cache.
The warm-up runs the requested steps and then continues until the clocks have been under
load for --warm-seconds (a short warm-up under-reports); the JSON says how long it ran.

The per-kernel split comes from a second pass over the same inputs that launches the two
halves through their own entry points (conv1d_causal4, then rglru_lru, whose interval also
holds the look-back status fill it launches first), with HIP events on the library's
stream (the torch current stream) around each launch; medians are reported, and the
roofline uses the average launch duration of the fused kernel.

Further legs (--no-extras skips them): the long-sequence forward (B=2, T=32768, D=4096),
the tiny fp32 forward's latency, 1024 decode steps at B=256, the fwd+bwd training workload
(B=4, T=2048, D=5376), the next rows (recurrent block, gated MLP, local MQA), the unfused
gates + scan split, prefill/decode latency tables.  The CPU oracle is timed per workload
on bounded samples (stated in the output).

Prints ONE JSON line.  With --gpus N > 1 it exits with a message: the build runs on one
GPU (no cross-GPU path exists).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "RG-LRU block tokens/sec + achieved HBM GB/s (B=8,T=2048,D_RNN=2560 bf16)"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
LRU_PROFILE = os.path.join(ROOT, "profiles", "lru_fused_train_fwd_B8_T2048_D2560_pmc.md")
LRU_SOURCES = [os.path.join(ROOT, "gated_linear_rnn_amd", "csrc", f)
               for f in ("lru.hip", "gemm_core.h", "rglru_device.h")]


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--warm-seconds", type=float, default=1.0,
                    help="keep warming up after --warmup steps until this much time has passed")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-extras", action="store_true", help="skip the decode and fwd+bwd timings")
    ap.add_argument("--split-only", action="store_true",
                    help="only time the unfused path (rglru_gates, then rglru_scan) and print "
                         "its figures (for kernel profiles of the scan)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only time the decode extra (1024 steps at B=256, eager and one graph) "
                         "and print its figures (for kernel profiles of the decode step)")
    ap.add_argument("--bwd-only", action="store_true",
                    help="only time the fwd+bwd extra (rglru_fwd + rglru_bwd at B=4, T=2048, "
                         "D=5376) and print its figures (for kernel profiles of the backward)")
    ap.add_argument("--long-only", action="store_true",
                    help="only time the long-sequence forward (B=2, T=32768, D=4096)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter calibration)")
    return ap.parse_args()


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha256():
    """SHA-256 over the sources of the fused RG-LRU kernel (lru.hip, gemm_core.h,
    rglru_device.h, in that order)."""
    h = hashlib.sha256()
    for f in LRU_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def _lru_traffic():
    """HBM bytes per fused-kernel launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; otherwise None."""
    try:
        txt = open(LRU_PROFILE).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", txt, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n,
                      "launches": 3}))


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this build runs the RG-LRU "
              f"temporal branch on one GPU only (no cross-GPU path exists).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    import gated_linear_rnn_amd as g
    import workloads

    g.load()
    torch.cuda.set_device(0)
    if args.bwd_only:
        print(json.dumps(bench_fwd_bwd(g, torch, np, workloads)))
        return
    if args.decode_only:
        print(json.dumps(bench_decode(g, torch, np, workloads)))
        return
    if args.split_only:
        print(json.dumps(bench_split(g, torch, np, workloads, measured_copy_gbps(torch))))
        return
    if args.long_only:
        print(json.dumps(bench_long(g, torch, np, workloads)))
        return
    w = workloads.TRAIN_FWD
    B, T, D = w.B, w.T, w.D
    M = B * T
    bf = torch.bfloat16
    dev = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt)

    _log("drawing inputs")
    p = workloads.make_inputs(w)
    xs = [dev(p["x"], bf)] + [dev(workloads.extra_inputs_x(w, k), bf) for k in (1, 2)]
    conv_w, conv_b = dev(p["conv_w"], bf), dev(p["conv_b"])
    W_a, W_x = dev(p["W_a"], bf), dev(p["W_x"], bf)
    b_a, b_x, lam = dev(p["b_a"]), dev(p["b_x"]), dev(p["lam"])
    u = torch.empty((B, T, D), dtype=bf, device="cuda")
    y = torch.empty((B, T, D), dtype=bf, device="cuda")
    hT = torch.empty((B, D), dtype=torch.float32, device="cuda")
    ws = g.workspace(g.fwd_workspace_bytes(B, T, D, bf))
    c = p["c"]

    def step(k):
        g.rglru_fwd(xs[k % len(xs)], conv_w, conv_b, None, W_a, W_x, b_a, b_x, lam, None, y, hT,
                    None, ws, c)

    warm_steps, warm_s = warm_up(torch, step, args.warmup, args.warm_seconds)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    _log(f"timing {args.steps} steps of rglru_fwd")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        evs[k][0].record()
        step(k)
        evs[k][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [e[0].elapsed_time(e[1]) for e in evs]
    tokens_per_s = M * args.steps / wall

    # per-kernel split: the same work through the two halves' entry points
    _log(f"per-kernel split: {args.steps} steps of conv1d_causal4 + rglru_lru")
    wsl = g.workspace(g.lru_workspace_bytes(B, T, D, bf))
    kev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for k in range(args.steps + 3):
        e = kev[k - 3] if k >= 3 else None
        if e is not None:
            e[0].record()
        g.conv1d_causal4(xs[k % len(xs)], conv_w, conv_b, None, u, None)
        if e is not None:
            e[1].record()
        g.rglru_lru(u, W_a, W_x, b_a, b_x, lam, None, y, hT, wsl, c)
        if e is not None:
            e[2].record()
    torch.cuda.synchronize()
    conv_l = [e[0].elapsed_time(e[1]) for e in kev]
    lru_l = [e[1].elapsed_time(e[2]) for e in kev]
    conv_ms, lru_ms = float(np.median(conv_l)), float(np.median(lru_l))
    # the roofline's launch duration: the mean interval of rglru_lru in this pass, where it
    # alternates with the conv as in the step (launched back to back, the kernel runs ~7%
    # slower: the clock drops under uninterrupted matrix-core load)
    lru_avg = float(np.mean(lru_l))

    gemm_flop = 2.0 * M * (2 * D) * D
    lru_tflops = gemm_flop / (lru_avg * 1e-3) / 1e12
    block_bytes = M * D * (2 + 2) + 2 * D * D * 2      # x in, y out, W_a and W_x once
    block_gbps = block_bytes / (wall / args.steps) / 1e9
    conv_bytes = M * D * (2 + 2)
    lru_bytes = M * D * (2 + 2 + 2) + 2 * D * D * 2    # u (GEMM operand), u (scan), y, W once
    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_steps,
        "warmup_s": warm_s,
        "ms_per_step": wall * 1e3 / args.steps,
        "ms_per_step_median_events": float(np.median(step_ms)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "T": T, "D_RNN": D, "io": "bf16",
                   "scan_state": "fp32", "c": c, "entry_point": "rglru_fwd"},
        "roofline": {
            "kernel": "lru_fused_kernel (gate GEMM + gates + chunked scan)",
            "bound": "mfma", "achieved": lru_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": lru_tflops / PEAK_BF16_TFLOPS, "traffic": _lru_traffic(),
            "flop_per_launch": gemm_flop, "avg_launch_ms": lru_avg,
            "median_launch_ms": lru_ms, "launches_timed": args.steps,
            "note": "mean event interval of rglru_lru calls alternating with conv1d_causal4; "
                    "each call also launches the look-back status fill (about 4.5 us) first",
        },
        "hbm": {
            "block_achieved_GBps": block_gbps,
            "block_bytes_per_step": block_bytes,
            "block_frac_of_peak": block_gbps / PEAK_HBM_GBPS,
            "conv_kernel_GBps": conv_bytes / (conv_ms * 1e-3) / 1e9,
            "lru_kernel_GBps": lru_bytes / (lru_ms * 1e-3) / 1e9,
            "peak_GBps": PEAK_HBM_GBPS,
        },
        "per_kernel_ms_median": {"conv": conv_ms, "lru_fused": lru_ms},
        "block_tokens_per_s_kernels": M / ((conv_ms + lru_ms) * 1e-3),
    }
    del xs, u, y, ws, wsl
    torch.cuda.empty_cache()
    copy_gbps = measured_copy_gbps(torch)
    out["hbm"]["measured_copy_GBps"] = copy_gbps
    out["hbm"]["block_frac_of_measured_copy"] = block_gbps / copy_gbps

    if not args.no_extras:
        out["long_fwd"] = bench_long(g, torch, np, workloads)
        out["tiny_fwd_f32"] = bench_tiny(g, torch, np, workloads)
        out["decode"] = bench_decode(g, torch, np, workloads)
        out["train_fwd_bwd"] = bench_fwd_bwd(g, torch, np, workloads)
        out["recurrent_block_fwd"] = bench_block(g, torch, np, workloads)
        out["prefill_decode_latency"] = bench_latency(g, torch, np, workloads)
        out["gated_mlp_fwd"] = bench_mlp(g, torch, np, workloads)
        out["local_mqa_fwd"] = bench_mqa(g, torch, np, workloads)
        out["split_gates_scan"] = bench_split(g, torch, np, workloads, copy_gbps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p, np)
        out["cpu_baseline_per_workload"] = cpu_baseline_per_workload(np, workloads)
    print(json.dumps(out))


def warm_up(torch, step, steps, seconds):
    """Run `steps` steps, then keep going until `seconds` have passed (synchronising every
    25 steps so the clock measures GPU time).  Returns (steps run, seconds)."""
    _log(f"warmup: {steps} steps, then until {seconds:.1f} s")
    t0 = time.perf_counter()
    n = 0
    while n < steps or time.perf_counter() - t0 < seconds:
        step(n)
        n += 1
        if n % 25 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n, time.perf_counter() - t0


def bench_long(g, torch, np, workloads, steps=10):
    """The long-sequence forward, B=2, T=32768, D=4096 (a^c in [0.999, 0.9999], h0 ~ N(0,1)):
    rglru_fwd per call (median of `steps` after a timed warm-up), and the per-kernel split
    through conv1d_causal4 + rglru_lru with events."""
    w = workloads.LONG_FWD
    B, T, D = w.B, w.T, w.D
    M = B * T
    bf = torch.bfloat16
    dev = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt)
    _log(f"long forward {B}x{T}x{D}: drawing inputs")
    p = workloads.make_inputs(w)
    x = dev(p["x"], bf)
    cw, cb = dev(p["conv_w"], bf), dev(p["conv_b"])
    Wa, Wx, ba, bx, lam = dev(p["W_a"], bf), dev(p["W_x"], bf), dev(p["b_a"]), dev(p["b_x"]), dev(p["lam"])
    h0 = dev(p["h0"])
    del p
    y = torch.empty_like(x)
    hT = torch.empty((B, D), dtype=torch.float32, device="cuda")
    ws = g.workspace(g.fwd_workspace_bytes(B, T, D, bf))
    fwd = lambda k: g.rglru_fwd(x, cw, cb, None, Wa, Wx, ba, bx, lam, h0, y, hT, None, ws, 8.0)
    warm_up(torch, fwd, 3, 0.5)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for k in range(steps):
        evs[k][0].record()
        fwd(k)
        evs[k][1].record()
    torch.cuda.synchronize()
    fwd_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    u = torch.empty_like(x)
    wsl = g.workspace(g.lru_workspace_bytes(B, T, D, bf))
    for k in range(steps):
        evs[k][0].record()
        g.conv1d_causal4(x, cw, cb, None, u, None)
        evs[k][1].record()
        g.rglru_lru(u, Wa, Wx, ba, bx, lam, h0, y, hT, wsl, 8.0)
        evs[k][2].record()
    torch.cuda.synchronize()
    conv_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    lru_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    flop = 2.0 * M * (2 * D) * D
    block_bytes = M * D * (2 + 2) + 2 * D * D * 2
    out = {"workload": w.name, "steps": steps, "ms_per_call_median": fwd_ms,
           "tokens_per_s": M / (fwd_ms * 1e-3),
           "per_kernel_ms_median": {"conv": conv_ms, "lru_fused": lru_ms},
           "lru_TFLOPs": flop / (lru_ms * 1e-3) / 1e12,
           "lru_frac_of_bf16_peak": flop / (lru_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
           "flop_per_call": flop,
           "block_GBps": block_bytes / (fwd_ms * 1e-3) / 1e9,
           "conv_GBps": M * D * 4 / (conv_ms * 1e-3) / 1e9}
    del x, y, u, ws, wsl
    torch.cuda.empty_cache()
    return out


def bench_tiny(g, torch, np, workloads, steps=200):
    """The tiny fp32 forward (B=1, T=256, D=256): latency of one rglru_fwd call (median of
    `steps` calls, each bracketed by events)."""
    w = workloads.TINY_F32
    p = workloads.make_inputs(w)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    x, cw, cb = dev(p["x"]), dev(p["conv_w"]), dev(p["conv_b"])
    Wa, Wx, ba, bx, lam = dev(p["W_a"]), dev(p["W_x"]), dev(p["b_a"]), dev(p["b_x"]), dev(p["lam"])
    y = torch.empty_like(x)
    hT = torch.empty((w.B, w.D), device="cuda")
    ws = g.workspace(g.fwd_workspace_bytes(w.B, w.T, w.D, torch.float32))
    fwd = lambda k=0: g.rglru_fwd(x, cw, cb, None, Wa, Wx, ba, bx, lam, None, y, hT, None, ws, 8.0)
    for _ in range(20):
        fwd()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    lat = []
    for _ in range(steps):
        e0.record()
        fwd()
        e1.record()
        torch.cuda.synchronize()
        lat.append(e0.elapsed_time(e1))
    ms = float(np.median(lat))
    return {"workload": w.name, "calls": steps, "us_per_call_median": ms * 1e3,
            "tokens_per_s": w.B * w.T / (ms * 1e-3)}


def measured_copy_gbps(torch, nbytes=1 << 30, reps=20):
    """Device-to-device copy of a 1 GiB buffer (read + write bytes over the copy time):
    the achievable HBM bandwidth the block's algorithmic GB/s is also compared with."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2.0 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return gbps


def bench_decode(g, torch, np, workloads):
    """1024 dependent decode steps at B=256, D=2560 (eager launches and one hipGraph)."""
    w = workloads.DECODE.with_shape(T=64)     # 64 distinct seeded tokens, cycled
    p = workloads.make_inputs(w)
    bf = torch.bfloat16
    dev = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt)
    B, D, steps = w.B, w.D, workloads.DECODE.T
    toks = dev(p["x"], bf)
    cw, cb = dev(p["conv_w"], bf), dev(p["conv_b"])
    Wa, Wx, ba, bx, lam = dev(p["W_a"], bf), dev(p["W_x"], bf), dev(p["b_a"]), dev(p["b_x"]), dev(p["lam"])
    hist0, h0 = dev(p["conv_state"], bf), dev(p["h0"])
    hist, h = hist0.clone(), h0.clone()
    y = torch.empty((B, D), dtype=bf, device="cuda")
    ws = g.workspace(g.decode_workspace_bytes(B, D, bf))

    def run():
        for t in range(steps):
            g.rglru_decode_step(toks[t % w.T], cw, cb, hist, Wa, Wx, ba, bx, lam, h, y, ws, p["c"])

    reps = 3
    _log("decode: eager")
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    eager = []
    for _ in range(reps):
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        eager.append(e0.elapsed_time(e1))
    _log("decode: graph")
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    graph.replay()
    torch.cuda.synchronize()
    graphed = []
    for _ in range(reps):
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        graphed.append(e0.elapsed_time(e1))
    eager_ms, graph_ms = float(np.median(eager)), float(np.median(graphed))
    state_bytes = B * D * (4 + 4 + 6 + 6 + 2 + 2)   # h r/w, history r/w, x_t, y_t
    w_bytes = 2 * D * D * 2
    best = min(eager_ms, graph_ms)
    return {
        "workload": workloads.DECODE.name, "steps": steps,
        "tokens_per_s_eager": B * steps / (eager_ms * 1e-3),
        "tokens_per_s_graph": B * steps / (graph_ms * 1e-3),
        "us_per_step_eager": eager_ms * 1e3 / steps, "us_per_step_graph": graph_ms * 1e3 / steps,
        "state_update_GBps": state_bytes * steps / (best * 1e-3) / 1e9,
        "state_plus_weights_GBps": (state_bytes + w_bytes) * steps / (best * 1e-3) / 1e9,
        "runs": reps, "statistic": "median over runs of 1024 dependent steps",
        "note": "W (26 MB) and the state (16 MB) stay resident in the 256 MB Infinity Cache",
    }


def bench_fwd_bwd(g, torch, np, workloads):
    """rglru_fwd + rglru_bwd on the fwd+bwd training workload B=4, T=2048, D=5376."""
    w = workloads.TRAIN_BWD
    p = workloads.make_inputs(w)
    bf = torch.bfloat16
    dev = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt)
    B, T, D = w.B, w.T, w.D
    x, dy = dev(p["x"], bf), dev(p["dy"], bf)
    cw, cb = dev(p["conv_w"], bf), dev(p["conv_b"])
    Wa, Wx, ba, bx, lam = dev(p["W_a"], bf), dev(p["W_x"], bf), dev(p["b_a"]), dev(p["b_x"]), dev(p["lam"])
    wsf = g.workspace(g.fwd_workspace_bytes(B, T, D, bf))
    wsb = g.workspace(g.bwd_workspace_bytes(B, T, D, bf))
    _log("fwd+bwd")

    def once():
        y, hT, _ = g.forward(x, cw, cb, None, Wa, Wx, ba, bx, lam, None, p["c"], ws=wsf)
        e_mid.record()
        g.backward(x, cw, cb, None, Wa, Wx, ba, bx, lam, None, dy, None, p["c"], ws=wsb)

    e0, e_mid, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    for _ in range(5):
        once()
    torch.cuda.synchronize()
    fwd, bwd = [], []
    for _ in range(20):
        e0.record()
        once()
        e1.record()
        torch.cuda.synchronize()
        fwd.append(e0.elapsed_time(e_mid))
        bwd.append(e_mid.elapsed_time(e1))
    f, b = float(np.median(fwd)), float(np.median(bwd))
    del wsf, wsb
    # the training pair that keeps the forward's activations: rglru_fwd_train writes u, r, i
    # and every h_t, and rglru_bwd_saved starts from them instead of evaluating the forward
    wst = g.workspace(g.fwd_train_workspace_bytes(B, T, D, bf))
    wss = g.workspace(g.bwd_saved_workspace_bytes(B, T, D, bf))
    saved = g.workspace(g.train_saved_bytes(B, T, D, bf))

    def once_saved():
        g.forward_train(x, cw, cb, None, Wa, Wx, ba, bx, lam, None, p["c"], ws=wst, saved=saved)
        e_mid.record()
        g.backward(x, cw, cb, None, Wa, Wx, None, None, lam, None, dy, None, p["c"], ws=wss,
                   saved=saved)

    for _ in range(5):
        once_saved()
    torch.cuda.synchronize()
    fwd_s, bwd_s = [], []
    for _ in range(20):
        e0.record()
        once_saved()
        e1.record()
        torch.cuda.synchronize()
        fwd_s.append(e0.elapsed_time(e_mid))
        bwd_s.append(e_mid.elapsed_time(e1))
    fs, bs = float(np.median(fwd_s)), float(np.median(bwd_s))
    return {"workload": w.name, "fwd_ms": f, "bwd_ms": b, "runs": len(fwd), "statistic": "median",
            "tokens_per_s_fwd_bwd": B * T / ((f + b) * 1e-3),
            "saved_activations": {
                "fwd_train_ms": fs, "bwd_saved_ms": bs,
                "tokens_per_s_fwd_bwd": B * T / ((fs + bs) * 1e-3),
                "saved_bytes": g.train_saved_bytes(B, T, D, bf),
                "note": "rglru_fwd_train keeps u, r, i and every h_t; rglru_bwd_saved reads them "
                        "instead of evaluating the forward again (same gradients, bit for bit)"}}


def bench_block(g, torch, np, workloads, steps=50):
    """rglru_block_fwd (input linears + GeLU branch + conv + RG-LRU + product + output
    linear) at B=8, T=2048, D = D_RNN = 2560, bf16, inputs resident, warm clocks."""
    w = workloads.TRAIN_FWD
    p = workloads.make_block_inputs(w)
    bf = torch.bfloat16
    dev = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt)
    B, T, R = w.B, w.T, w.D
    D = p["d_model"]
    xb, W_in, W_out = dev(p["x_block"], bf), dev(p["W_in"], bf), dev(p["W_out"], bf)
    cw, cb = dev(p["conv_w"], bf), dev(p["conv_b"])
    Wa, Wx, ba, bx, lam = dev(p["W_a"], bf), dev(p["W_x"], bf), dev(p["b_a"]), dev(p["b_x"]), dev(p["lam"])
    out = torch.empty_like(xb)
    hT = torch.empty((B, R), dtype=torch.float32, device="cuda")
    ws = g.workspace(g.block_fwd_workspace_bytes(B, T, D, R, bf))
    _log("recurrent block")

    def once():
        g.rglru_block_fwd(xb, W_in, cw, cb, None, Wa, Wx, ba, bx, lam, None, W_out, out, hT, None,
                          ws, p["c"])

    for _ in range(steps):
        once()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        once()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    M = B * T
    flop = 2.0 * M * (2 * R * D + 2 * R * R + D * R)
    # decode steps of the whole block (rglru_block_decode_step), state carried in place
    dec = []
    gen = torch.Generator(device="cuda").manual_seed(3)
    for Bd in (1, 64, 256):
        xt = torch.randn((Bd, D), generator=gen, device="cuda").to(bf)
        cs = torch.randn((Bd, 3, R), generator=gen, device="cuda").to(bf)
        h = torch.randn((Bd, R), generator=gen, device="cuda")
        o = torch.empty((Bd, D), dtype=bf, device="cuda")
        wsd = g.workspace(g.block_decode_workspace_bytes(Bd, D, R, bf))
        step = lambda: g.rglru_block_decode_step(xt, W_in, cw, cb, cs, Wa, Wx, ba, bx, lam, h, W_out, o,
                                                 wsd, p["c"])
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(100):
            step()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 10.0
        dec.append({"B": Bd, "us_per_step": us, "tokens_per_s": Bd / (us * 1e-6)})
    return {"workload": f"block_fwd_bf16_B{B}_T{T}_D{D}_R{R}", "ms_per_step": ms,
            "tokens_per_s": M / (ms * 1e-3), "TFLOPs": flop / (ms * 1e-3) / 1e12,
            "flop_per_step": flop, "steps": steps, "decode_step": dec}


def bench_mlp(g, torch, np, workloads, steps=30):
    """gated_mlp_fwd (two D -> 3D linears, GeLU product, 3D -> D linear) at B=8, T=2048,
    D=2560, bf16, inputs resident, warm clocks."""
    w = workloads.TRAIN_FWD
    p = workloads.make_mlp_inputs(w)
    bf = torch.bfloat16
    dev = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt)
    x, W1, W2, W3 = (dev(p[k], bf) for k in ("x", "W_1", "W_2", "W_3"))
    B, T, D = w.B, w.T, w.D
    MD = W1.shape[0]
    out = torch.empty_like(x)
    ws = g.workspace(g.mlp_fwd_workspace_bytes(B, T, D, MD, bf))
    _log("gated MLP")
    for _ in range(steps):
        g.gated_mlp_fwd(x, W1, W2, W3, out, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.gated_mlp_fwd(x, W1, W2, W3, out, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    M = B * T
    flop = 2.0 * M * (2 * MD * D + MD * D)
    return {"workload": f"mlp_fwd_bf16_B{B}_T{T}_D{D}_MD{MD}", "ms_per_step": ms,
            "tokens_per_s": M / (ms * 1e-3), "TFLOPs": flop / (ms * 1e-3) / 1e12,
            "flop_per_step": flop, "steps": steps}


def bench_mqa(g, torch, np, workloads, steps=30, window=1024):
    """local_mqa_fwd (q/k/v projections with RoPE, sliding-window attention, output
    projection) at B=8, T=2048, D=2560 (20 heads of 128), window 1024, bf16."""
    w = workloads.TRAIN_FWD
    p = workloads.make_mqa_inputs(w, window)
    bf = torch.bfloat16
    dev = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt)
    B, T, D = w.B, w.T, w.D
    x = dev(p["x"], bf)
    Wqkv = dev(np.concatenate([p["W_q"], p["W_k"], p["W_v"]]), bf)
    Wo = dev(p["W_o"], bf)
    out = torch.empty_like(x)
    ws = g.workspace(g.mqa_fwd_workspace_bytes(B, T, D, bf))
    _log("local MQA")
    run = lambda: g.local_mqa_fwd(x, Wqkv, Wo, out, None, None, ws, window, 0)
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # decode steps with a full window of cached keys (position 2047), one per batch size
    dec = []
    gen = torch.Generator(device="cuda").manual_seed(5)
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for Bd in (1, 64, 256):
        kc = torch.randn((Bd, window, 128), generator=gen, device="cuda").to(bf)
        vc = torch.randn((Bd, window, 128), generator=gen, device="cuda").to(bf)
        xt = torch.randn((Bd, D), generator=gen, device="cuda").to(bf)
        pos = torch.full((Bd,), 2047, dtype=torch.int32, device="cuda")
        o = torch.empty((Bd, D), dtype=bf, device="cuda")
        wsd = g.workspace(g.mqa_decode_workspace_bytes(Bd, D, bf))
        step = lambda: g.local_mqa_decode_step(pos, xt, Wqkv, Wo, kc, vc, o, wsd)
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        e2.record()
        for _ in range(100):
            step()
        e3.record()
        torch.cuda.synchronize()
        us = e2.elapsed_time(e3) * 10.0
        dec.append({"B": Bd, "us_per_step": us, "tokens_per_s": Bd / (us * 1e-6),
                    "cache_bytes_per_sequence": 2 * window * 128 * 2})
        del kc, vc, wsd
    M, H = B * T, D // 128
    pairs = B * H * sum(min(t + 1, window) for t in range(T))     # (query, key) pairs
    attn_flop = 4.0 * 128 * pairs
    flop = 2.0 * M * D * (D + 256) + attn_flop + 2.0 * M * D * D
    return {"workload": f"mqa_fwd_bf16_B{B}_T{T}_D{D}_H{H}_W{window}", "ms_per_step": ms,
            "tokens_per_s": M / (ms * 1e-3), "TFLOPs": flop / (ms * 1e-3) / 1e12,
            "flop_per_step": flop, "attention_flop": attn_flop, "steps": steps,
            "decode_full_window": dec}


def bench_split(g, torch, np, workloads, copy_gbps, steps=50):
    """The unfused form of the same forward at the headline shape: rglru_gates (the gate GEMM
    writing a and beta, fp32) then rglru_scan (the conv recomputed from x, the chunked scan,
    y), timed per kernel with events, then the scan alone, back to back.  The scan moves 12
    bytes per element (x 2, a 4, beta 4, y 2); its interval includes the look-back status
    fill it launches first."""
    w = workloads.TRAIN_FWD
    B, T, D = w.B, w.T, w.D
    bf = torch.bfloat16
    p = workloads.make_inputs(w)
    dev = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt)
    x, cw, cb = dev(p["x"], bf), dev(p["conv_w"], bf), dev(p["conv_b"])
    Wa, Wx, ba, bx, lam = dev(p["W_a"], bf), dev(p["W_x"], bf), dev(p["b_a"]), dev(p["b_x"]), dev(p["lam"])
    u = torch.empty_like(x)
    y = torch.empty_like(x)
    hT = torch.empty((B, D), dtype=torch.float32, device="cuda")
    a = torch.empty((B, T, D), dtype=torch.float32, device="cuda")
    beta = torch.empty_like(a)
    ws = g.workspace(g.scan_workspace_bytes(B, T, D, bf))
    g.conv1d_causal4(x, cw, cb, None, u, None)

    def once(ev=None):
        if ev is not None:
            ev[0].record()
        g.rglru_gates(u, Wa, Wx, ba, bx, lam, a, beta, p["c"])
        if ev is not None:
            ev[1].record()
        g.rglru_scan(x, cw, cb, None, a, beta, None, y, hT, ws)
        if ev is not None:
            ev[2].record()

    for _ in range(steps):
        once()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for k in range(steps):
        once(evs[k])
    torch.cuda.synchronize()
    gates_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    scan_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    scan_bytes = B * T * D * 12
    scan_gbps = scan_bytes / (scan_ms * 1e-3) / 1e9
    # the scan alone, back to back (no gates kernel writing a and beta just before)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.rglru_scan(x, cw, cb, None, a, beta, None, y, hT, ws)
    e1.record()
    torch.cuda.synchronize()
    alone_ms = e0.elapsed_time(e1) / steps
    alone_gbps = scan_bytes / (alone_ms * 1e-3) / 1e9
    gflop = 2.0 * B * T * 2 * D * D
    return {
        "workload": w.name,
        "gates_ms": gates_ms,
        "gates_TFLOPs": gflop / (gates_ms * 1e-3) / 1e12,
        "scan_ms": scan_ms,
        "scan_bytes": scan_bytes,
        "scan_GBps": scan_gbps,
        "scan_frac_of_peak": scan_gbps / PEAK_HBM_GBPS,
        "scan_frac_of_measured_copy": scan_gbps / copy_gbps,
        "scan_alone_ms": alone_ms,
        "scan_alone_GBps": alone_gbps,
        "scan_alone_frac_of_peak": alone_gbps / PEAK_HBM_GBPS,
        "tokens_per_s_gates_plus_scan": B * T / ((gates_ms + scan_ms) * 1e-3),
        "steps": steps,
    }


def bench_latency(g, torch, np, workloads):
    """Prefill latency (one rglru_fwd call) by context length and batch, decode latency per
    step by batch, and the fixed state carried per sequence, at D = 2560 with the headline
    workload's parameters (the pages' checklist: prefill and decode latency by context
    length and batch size, state memory)."""
    w = workloads.TRAIN_FWD
    p = workloads.make_inputs(w.with_shape(B=1, T=1))
    bf = torch.bfloat16
    dev = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt)
    D = w.D
    cw, cb = dev(p["conv_w"], bf), dev(p["conv_b"])
    Wa, Wx, ba, bx, lam = dev(p["W_a"], bf), dev(p["W_x"], bf), dev(p["b_a"]), dev(p["b_x"]), dev(p["lam"])
    gen = torch.Generator(device="cuda").manual_seed(17)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    _log("prefill/decode latency")
    prefill = []
    for B in (1, 8, 32):
        for T in (512, 2048, 8192):
            x = torch.randn((B, T, D), generator=gen, device="cuda").to(bf)
            y = torch.empty_like(x)
            hT = torch.empty((B, D), device="cuda")
            cso = torch.empty((B, 3, D), dtype=bf, device="cuda")
            ws = g.workspace(g.fwd_workspace_bytes(B, T, D, bf))
            ms = timed(lambda: g.rglru_fwd(x, cw, cb, None, Wa, Wx, ba, bx, lam, None, y, hT, cso, ws,
                                           p["c"]), 10)
            prefill.append({"B": B, "T": T, "ms": ms, "tokens_per_s": B * T / (ms * 1e-3)})
            del x, y, ws
    decode = []
    for B in (1, 8, 64, 256):
        xt = torch.randn((B, D), generator=gen, device="cuda").to(bf)
        hist = torch.randn((B, 3, D), generator=gen, device="cuda").to(bf)
        h = torch.randn((B, D), generator=gen, device="cuda")
        yt = torch.empty((B, D), dtype=bf, device="cuda")
        ws = g.workspace(g.decode_workspace_bytes(B, D, bf))
        ms = timed(lambda: g.rglru_decode_step(xt, cw, cb, hist, Wa, Wx, ba, bx, lam, h, yt, ws,
                                               p["c"]), 200)
        decode.append({"B": B, "us_per_step": ms * 1e3, "tokens_per_s": B / (ms * 1e-3)})
    torch.cuda.empty_cache()
    return {"D": D, "prefill_rglru_fwd": prefill, "decode_step_eager": decode,
            "state_bytes_per_sequence": D * 4 + 3 * D * 2,
            "note": "the state (h fp32 + 3-token bf16 conv history) does not grow with context"}


def cpu_baseline(p, np, min_seconds=10.0):
    """The CPU oracle, as it stands, on a bounded sample of the same workload: its forward
    over the whole headline batch, repeated until at least min_seconds have passed."""
    import oracle
    Bs = p["x"].shape[0]
    cores = len(os.sched_getaffinity(0))
    _log(f"cpu baseline: oracle forward on {Bs} sequences ({cores} cores)")
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(p["x"][:Bs], p["conv_w"], p["conv_b"], None, p["W_a"], p["W_x"], p["b_a"],
                       p["b_x"], p["lam"], None, p["c"], "bf16")
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    T = p["x"].shape[1]
    return {"value": reps * Bs * T / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"oracle forward (fp64 NumPy, BLAS threads = cores) over the whole "
                      f"{Bs}x{T}x{p['x'].shape[2]} workload, {reps} times ({reps * Bs * T} tokens, "
                      f"{dt:.1f} s)"}


def _timed(fn, min_seconds):
    """Run fn until min_seconds have passed; returns (runs, seconds)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            return reps, dt


def cpu_baseline_per_workload(np, workloads, min_seconds=4.0):
    """The CPU oracle, as it stands, on a bounded sample of each workload, in tokens/s (the
    sample of each is stated).  Every sample keeps the workload's D, distributions and
    weights; only batch rows, sequence length or decode steps are cut, which the oracle's
    cost scales with linearly (its GEMMs are per row, its recurrence per step)."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    out = {"cores": cores, "kind": "oracle", "unit": "tokens/s"}

    w = workloads.TINY_F32
    p = workloads.make_inputs(w)
    _log("cpu baseline: tiny forward")
    reps, dt = _timed(lambda: oracle.forward(p["x"], p["conv_w"], p["conv_b"], None, p["W_a"],
                                             p["W_x"], p["b_a"], p["b_x"], p["lam"], None, p["c"],
                                             "f32"), min_seconds)
    out[w.name] = {"value": reps * w.B * w.T / dt,
                   "sample": f"the whole workload, {reps} forwards in {dt:.1f} s"}

    w = workloads.DECODE
    steps = 8
    p = workloads.make_inputs(w.with_shape(T=steps))
    _log(f"cpu baseline: {steps} decode steps at B={w.B}")

    def dec():
        hist, h = p["conv_state"], p["h0"]
        for t in range(steps):
            y, hist, h = oracle.decode_step(p["x"][t], p["conv_w"], p["conv_b"], hist, p["W_a"],
                                            p["W_x"], p["b_a"], p["b_x"], p["lam"], h, p["c"], "bf16")
    reps, dt = _timed(dec, min_seconds)
    out[w.name] = {"value": reps * steps * w.B / dt,
                   "sample": f"{steps} of the 1024 dependent steps at B={w.B}, D={w.D}, "
                             f"{reps} times in {dt:.1f} s (the cost per step does not change "
                             f"with the step index)"}

    w = workloads.LONG_FWD
    Ts = 2048
    p = workloads.make_inputs(w.with_shape(B=1, T=Ts))
    _log(f"cpu baseline: long forward, one sequence of {Ts} steps")
    reps, dt = _timed(lambda: oracle.forward(p["x"], p["conv_w"], p["conv_b"], None, p["W_a"],
                                             p["W_x"], p["b_a"], p["b_x"], p["lam"], p["h0"],
                                             p["c"], "bf16"), min_seconds)
    out[w.name] = {"value": reps * Ts / dt,
                   "sample": f"one sequence of {Ts} of the {w.T} steps at D={w.D} (the "
                             f"workload's recipe), {reps} forwards in {dt:.1f} s"}

    w = workloads.TRAIN_BWD
    p = workloads.make_inputs(w.with_shape(B=1))
    _log("cpu baseline: fwd+bwd, one sequence")

    def fb():
        oracle.forward(p["x"], p["conv_w"], p["conv_b"], None, p["W_a"], p["W_x"], p["b_a"],
                       p["b_x"], p["lam"], None, p["c"], "bf16")
        oracle.backward(p["x"], p["conv_w"], p["conv_b"], None, p["W_a"], p["W_x"], p["b_a"],
                        p["b_x"], p["lam"], None, p["c"], "bf16", p["dy"])
    reps, dt = _timed(fb, min_seconds)
    out[w.name] = {"value": reps * w.T / dt,
                   "sample": f"one of the {w.B} sequences ({w.T} steps, D={w.D}), forward then "
                             f"backward, {reps} times in {dt:.1f} s"}
    return out


if __name__ == "__main__":
    main()
