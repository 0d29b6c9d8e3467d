"""Benchmark of the GLA forward on one MI355X.

One step = one chunked prefill (gla_prefill_chunked) of the headline workload:
B=8, H=16, L=4096, d_k=d_v=128, chunk 64, bf16 q/k/v, fp32 key-dimension log-gates,
final fp32 state written.  Inputs are drawn once (seeded, synthetic) and are resident
in HBM before the timed region.  The same run also times the recurrent decode
workload (B=256, H=32, d=128: a 512-token prefill fills the state, then 1024
gla_decode_step calls), and the fp64 CPU oracle on a bounded sample of the prefill
workload.

Prints ONE JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]

Profiling helpers (same file, so every profile command runs committed code only):
  --copy-kernel                 run only a plain device copy of known size (the
                                calibration kernel for the HBM byte counters)
  --summarize-stats DIR         turn a rocprofv3 --kernel-trace --stats run into a text
                                summary under profiles/
  --summarize-traffic F W CF CW turn four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE
                                of the prefill, then of the copy kernel) into the traffic
                                summary that the JSON line's roofline.traffic reads
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GLA prefill tokens/s + % MFMA peak (L=4096,d=128); decode tok/s + HBM GB/s"
HBM_PEAK_GBS = 8000.0                 # MI355X HBM3E, GB/s (datasheet)
BF16_MFMA_PEAK_TFLOPS = 2516.6        # dense bf16 MFMA, TFLOP/s (256 CU x 4096 flop/clk x 2.4 GHz)


PROFILES = os.path.join(ROOT, "profiles")
PREFILL_KERNEL = "prefill_kernel"
PREFILL_SOURCES = ("gla_prefill.hpp", "gla_prefill_inst.hip", "gla_device.hpp", "gla_launch.hpp", "gla_slow.hpp")
TRAFFIC_FILE = os.path.join(PROFILES, "prefill_kernel_bf16_dk128_L4096_traffic.txt")
STATS_FILE = os.path.join(PROFILES, "gla_kernels_bench_workloads_kernel_stats.txt")
COPY_MIB = 512                        # calibration copy: reads and writes this many MiB


def prefill_bytes(B, H, L, dk, dv, es=2, gate="keydim"):
    """Algorithmic HBM bytes of one prefill: read q, k, v, g once, write o and the final
    state once (per token-head 3*d*es + 4*d_k + d*es; per head d_k*d_v*4)."""
    g = 4 * dk if gate == "keydim" else (4 if gate == "scalar" else 0)
    return B * H * (L * (2 * dk * es + dv * es + g + dv * es) + dk * dv * 4)


def prefill_flops(B, H, L, dk, dv, C):
    """Causal-count flops: per chunk C(C+1)(d_k+d_v) for the masked score and value
    products plus 4 C d_k d_v for the state update and the inter-chunk read-out."""
    n_full, tail = divmod(L, C)
    per = lambda c: c * (c + 1) * (dk + dv) + 4 * c * dk * dv
    return B * H * (n_full * per(C) + (per(tail) if tail else 0))


def delta_bytes(B, H, L, dk, dv, es=2):
    """Algorithmic HBM bytes of one delta-rule prefill: read q, k, v and beta once, write
    o and the final state once (the workspace between its two kernels not counted)."""
    return B * H * (L * (2 * dk * es + dv * es + 4 + dv * es) + dk * dv * 4)


def delta_flops(B, H, L, dk, dv, C):
    """Flops of the chunkwise delta rule, causal count: per chunk of c tokens the
    strictly lower K K^T (c(c-1) d_k), the triangular inverse (c^3 / 3), W and U~ from
    the lower-triangular inverse (c(c+1)(d_k + d_v)), the masked scores and their
    product with U (c(c+1)(d_k + d_v)), and the three state products U~ - W S, Q S and
    S += K^T U (6 c d_k d_v)."""
    n_full, tail = divmod(L, C)
    per = lambda c: c * (c - 1) * dk + c ** 3 // 3 + 2 * c * (c + 1) * (dk + dv) + 6 * c * dk * dv
    return B * H * (n_full * per(C) + (per(tail) if tail else 0))


def decode_step_bytes(B, H, dk, dv, es=2):
    """Per step: read + write the fp32 state, read q, k, v, g, write o."""
    return B * H * (2 * dk * dv * 4 + (2 * dk + dv) * es + 4 * dk + dv * es)


def _events_ms(fn, n, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(n):
        fn()
    stop.record(stream)
    stop.synchronize()
    return start.elapsed_time(stop)


PEAKS_SRC = os.path.join(ROOT, "bench_peaks.hip")
PEAKS_LIB = os.path.join(ROOT, "bench_peaks.so")


def build_peaks():
    """Compile bench_peaks.hip (achievable-peak kernels for this report) for gfx950."""
    import subprocess
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc"
    cmd = [hipcc, "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", PEAKS_SRC, "-o", PEAKS_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for bench_peaks.hip:\n" + r.stdout + r.stderr)
    return PEAKS_LIB


def achievable_peaks():
    """This card's achievable HBM rate for the prefill's traffic mix and dense bf16
    matrix-core rate, measured now (bench_peaks.hip); None where unavailable."""
    import ctypes
    out = {"hbm_GBs": None, "hbm_inplace_GBs": None, "mfma_bf16_tflops": None,
           "note": "bench_peaks.hip: a streaming kernel with the prefill's read:write mix (5:1, "
                   "non-temporal 16-byte accesses), an in-place non-temporal scaling of 512 MiB (the "
                   "decode step's pattern) and a loop of independent bf16 16x16x32 products"}
    if not os.path.exists(PEAKS_LIB):
        out["note"] += "; not built"
        return out
    lib = ctypes.CDLL(PEAKS_LIB)
    for name, key in (("peaks_stream", "hbm_GBs"), ("peaks_inplace", "hbm_inplace_GBs"),
                      ("peaks_mfma", "mfma_bf16_tflops")):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.POINTER(ctypes.c_double)]
        v = ctypes.c_double(0.0)
        if fn(ctypes.byref(v)) == 0:
            out[key] = v.value
    return out


def _cold_ms(torch, step, stream, n, flush):
    """Median per-launch time of ``step`` with the caches flushed before each launch:
    ``flush`` (a 1 GiB device buffer) is overwritten outside the timed interval, which
    evicts the L2 caches and the 256 MB last-level cache."""
    times = []
    for _ in range(n):
        flush.fill_(1.0)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    return times[len(times) // 2]


def _settle(torch, step, seconds):
    """Untimed launches of ``step`` for at least ``seconds`` (one at a time), so that a
    workload is timed in its steady state: the first launches after a switch of
    workload and inputs run measurably slower."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        step()
        torch.cuda.synchronize()


def run_prefill(args, torch, api, inputs):
    w = inputs.WORKLOADS["gla_prefill"]
    inp = inputs.draw(w, device="cuda")
    o = torch.empty(w.B, w.H, w.L, w.d_v, dtype=w.dtype, device="cuda")
    s = torch.empty(w.B, w.H, w.d_k, w.d_v, dtype=torch.float32, device="cuda")
    ws_n = api.workspace_bytes(w.B, w.H, w.L, w.d_k, w.d_v, w.chunk, w.dtype)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda") if ws_n else None
    stream = torch.cuda.current_stream()

    def step():
        api.prefill(inp["q"], inp["k"], inp["v"], log_gate=inp["g"], gate="keydim", chunk=w.chunk,
                    out=o, final_state=s, workspace=ws, stream=stream)

    # untimed: launches until the clocks have settled (at least --settle-s seconds),
    # then the W warm-up steps of the contract
    settle = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(20):
            step()
        settle += 20
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = _events_ms(step, args.steps, stream)          # the kernel runs on this stream
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = ms / args.steps
    # after the timed region: the same number of launches, each between its own pair of
    # events (back to back on the stream), for the spread of single-launch times
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    one = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    launch_stats = {"launches": len(one), "min_ms": one[0], "median_ms": one[len(one) // 2],
                    "p90_ms": one[min(len(one) - 1, (9 * len(one)) // 10)]}
    flush = torch.empty(2**28, dtype=torch.float32, device="cuda")
    launch_stats["cold_median_ms"] = _cold_ms(torch, step, stream, 15, flush)
    del flush
    nbytes = prefill_bytes(w.B, w.H, w.L, w.d_k, w.d_v)
    flops = prefill_flops(w.B, w.H, w.L, w.d_k, w.d_v, w.chunk)
    return dict(w=w, inp=inp, ms_per_step=per, wall_s=wall, bytes=nbytes, flops=flops,
                settle_launches=settle, launch_stats=launch_stats)


def run_other_prefills(args, torch, api, inputs, baselines=None):
    """The other prefill workloads, timed the same way (reported beside the headline;
    fewer steps), each also with the caches flushed before every launch.  Bytes follow
    the same convention as the headline workload.  With ``baselines`` (a dict), the
    oracle is timed on each workload's inputs too (cpu_baseline_prefill)."""
    out = {}
    for name in ("linear_elu1", "scalar_long", "fp32_single_head"):
        w = inputs.WORKLOADS[name]
        inp = inputs.draw(w, device="cuda")
        o = torch.empty(w.B, w.H, w.L, w.d_v, dtype=w.dtype, device="cuda")
        s = torch.empty(w.B, w.H, w.d_k, w.d_v, dtype=torch.float32, device="cuda")
        # the segmented workloads' workspace, allocated once as a caller running many
        # prefills would (as for the headline)
        ws_n = api.workspace_bytes(w.B, w.H, w.L, w.d_k, w.d_v, w.chunk, w.dtype)
        ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda") if ws_n else None
        stream = torch.cuda.current_stream()

        def step():
            api.prefill(inp["q"], inp["k"], inp["v"], log_gate=inp["g"], gate=w.gate, chunk=w.chunk,
                        feature_map=w.feature_map, out=o, final_state=s, workspace=ws, stream=stream)

        _settle(torch, step, args.settle_s / 4)
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        n = max(5, args.steps // 2)
        per = _events_ms(step, n, stream) / n
        es = 2 if w.dtype == torch.bfloat16 else 4
        nbytes = prefill_bytes(w.B, w.H, w.L, w.d_k, w.d_v, es=es, gate=w.gate or "none")
        gbs = nbytes / (per / 1e3) / 1e9
        flush = torch.empty(2**28, dtype=torch.float32, device="cuda")
        cold = _cold_ms(torch, step, stream, 15, flush)
        del flush
        if baselines is not None:
            baselines[name] = cpu_baseline_prefill(w, inp, args.cpu_budget_s / 5)
        out[name] = {"ms_per_step": per, "ms_per_step_cold": cold, "tokens_per_s": w.B * w.L / (per / 1e3),
                     "GB_per_s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS, "bytes_per_launch": nbytes,
                     "shape": "B=%d H=%d L=%d d_k=%d d_v=%d chunk=%d %s gate=%s phi=%s" % (
                         w.B, w.H, w.L, w.d_k, w.d_v, w.chunk, str(w.dtype).replace("torch.", ""), w.gate,
                         w.feature_map or "identity")}
        del inp, o, s, ws
    # the normalised form (normaliser state z beside S) at the headline shape, elu+1
    w = inputs.WORKLOADS["gla_prefill"]
    inp = inputs.draw(w, device="cuda")
    o = torch.empty(w.B, w.H, w.L, w.d_v, dtype=w.dtype, device="cuda")
    s = torch.empty(w.B, w.H, w.d_k, w.d_v, dtype=torch.float32, device="cuda")
    z = torch.empty(w.B, w.H, w.d_k, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step_norm():
        api.prefill_norm(inp["q"], inp["k"], inp["v"], log_gate=inp["g"], gate="keydim", chunk=w.chunk,
                         feature_map="elu1", out=o, final_state=s, final_norm=z, stream=stream)

    _settle(torch, step_norm, args.settle_s / 4)
    for _ in range(3):
        step_norm()
    torch.cuda.synchronize()
    n = max(5, args.steps // 2)
    per = _events_ms(step_norm, n, stream) / n
    nbytes = prefill_bytes(w.B, w.H, w.L, w.d_k, w.d_v) + w.B * w.H * w.d_k * 4
    gbs = nbytes / (per / 1e3) / 1e9
    out["gla_prefill_norm_elu1"] = {
        "ms_per_step": per, "tokens_per_s": w.B * w.L / (per / 1e3), "GB_per_s": gbs,
        "hbm_frac": gbs / HBM_PEAK_GBS, "bytes_per_launch": nbytes,
        "shape": "B=%d H=%d L=%d d_k=%d d_v=%d chunk=%d bfloat16 gate=keydim phi=elu1, normalised" % (
            w.B, w.H, w.L, w.d_k, w.d_v, w.chunk)}
    return out


def run_decode(args, torch, api, inputs):
    w = inputs.WORKLOADS["decode"]
    pre = inputs.draw(w, device="cuda")
    _, state = api.prefill(pre["q"], pre["k"], pre["v"], log_gate=pre["g"], gate="keydim", chunk=w.chunk)
    T = args.decode_steps
    d = inputs.draw_decode(w, steps=T, device="cuda")
    # one head of every sequence, prompt then steps, for the oracle beside the decode
    bi = torch.arange(w.B, device="cuda")
    hi = (7 * bi) % w.H
    sample = {key: torch.cat([pre[key][bi, hi], d[key][:, bi, hi].transpose(0, 1)], dim=1).unsqueeze(1).cpu()
              for key in ("q", "k", "v", "g")}
    del pre
    o = torch.empty(w.B, w.H, w.d_v, dtype=w.dtype, device="cuda")
    stream = torch.cuda.current_stream()
    saved = state.clone()
    for t in range(min(3, T)):                           # warm-up steps, then restore
        api.decode_step(d["q"][t], d["k"][t], d["v"][t], log_gate=d["g"][t], state=state,
                        gate="keydim", out=o, stream=stream)
    state.copy_(saved)
    torch.cuda.synchronize()
    it = iter(range(T))

    def step():
        t = next(it)
        api.decode_step(d["q"][t], d["k"][t], d["v"][t], log_gate=d["g"][t], state=state,
                        gate="keydim", out=o, stream=stream)

    ms = _events_ms(step, T, stream)
    per = ms / T
    # single steps with the caches flushed before each (the 512 MiB state exceeds them
    # anyway; the step inputs do not)
    flush = torch.empty(2**28, dtype=torch.float32, device="cuda")
    it = iter(range(T))
    cold = _cold_ms(torch, step, stream, min(T, 15), flush)
    del flush
    nbytes = decode_step_bytes(w.B, w.H, w.d_k, w.d_v)
    # the normalised step (elu+1, normaliser state z updated beside S), fewer steps
    z = torch.ones(w.B, w.H, w.d_k, dtype=torch.float32, device="cuda")
    Tn = min(T, 256)
    it = iter(range(Tn))

    def step_norm():
        t = next(it)
        api.decode_step_norm(d["q"][t], d["k"][t], d["v"][t], log_gate=d["g"][t], state=state, norm=z,
                             gate="keydim", feature_map="elu1", out=o, stream=stream)

    per_n = _events_ms(step_norm, Tn, stream) / Tn
    nbytes_n = nbytes + w.B * w.H * w.d_k * 8
    return dict(w=w, steps=T, ms_per_step=per, ms_per_step_cold=cold, bytes=nbytes, norm_steps=Tn,
                norm_ms_per_step=per_n, norm_bytes=nbytes_n, oracle_sample=sample)


def run_delta(args, torch, api, inputs):
    """The delta rule ("Attention is recurrent", Delta attention): the chunkwise prefill
    at the gla_prefill shape and, at the decode shape, single-token steps."""
    w = inputs.WORKLOADS["delta_prefill"]
    inp = inputs.draw_delta(w, device="cuda")
    o = torch.empty(w.B, w.H, w.L, w.d_v, dtype=w.dtype, device="cuda")
    s = torch.empty(w.B, w.H, w.d_k, w.d_v, dtype=torch.float32, device="cuda")
    ws = torch.empty(api.delta_workspace_bytes(w.B, w.H, w.L, w.d_k, w.d_v, w.chunk, w.dtype),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        api.prefill_delta(inp["q"], inp["k"], inp["v"], inp["beta"], chunk=w.chunk, out=o, final_state=s,
                          workspace=ws, stream=stream)

    _settle(torch, step, args.settle_s / 4)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    n = max(5, args.steps // 2)
    per = _events_ms(step, n, stream) / n
    nbytes = delta_bytes(w.B, w.H, w.L, w.d_k, w.d_v)
    flops = delta_flops(w.B, w.H, w.L, w.d_k, w.d_v, w.chunk)
    gbs = nbytes / (per / 1e3) / 1e9
    tfl = flops / (per / 1e3) / 1e12
    out = {"prefill": {
        "workload": "delta_prefill: B=%d H=%d L=%d d_k=%d d_v=%d chunk=%d, bf16 q/k/v (unit-length q, k), "
                    "fp32 beta = sigmoid(N(0,1)), fp32 final state" % (w.B, w.H, w.L, w.d_k, w.d_v, w.chunk),
        "ms_per_step": per, "tokens_per_s": w.B * w.L / (per / 1e3), "GB_per_s": gbs,
        "hbm_frac": gbs / HBM_PEAK_GBS, "bytes_per_launch": nbytes, "tflops": tfl,
        "mfma_frac": tfl / BF16_MFMA_PEAK_TFLOPS, "flops_per_launch": flops,
        "workspace_bytes": int(ws.numel()),
        "kernels": ("delta_fused_kernel (each chunk's system solved beside the previous chunk's state update)"
                    if w.chunk <= 32 else
                    "delta_prep_kernel (all chunks in parallel) then delta_scan_kernel (chunks in order)")}}
    del inp, o, s, ws
    wd = inputs.WORKLOADS["decode"]
    T = min(256, args.decode_steps)
    d = inputs.draw_delta_decode(dataclass_replace(w, d_k=wd.d_k, d_v=wd.d_v), steps=T, B=wd.B, H=wd.H,
                                 device="cuda")
    state = inputs.draw_state(wd.B, wd.H, wd.d_k, wd.d_v, seed=17, scale=0.1, device="cuda")
    od = torch.empty(wd.B, wd.H, wd.d_v, dtype=torch.bfloat16, device="cuda")
    it = iter(range(T))

    def dstep():
        t = next(it)
        api.decode_step_delta(d["q"][t], d["k"][t], d["v"][t], d["beta"][t], state=state, out=od, stream=stream)

    torch.cuda.synchronize()
    dper = _events_ms(dstep, T, stream) / T
    dbytes = decode_step_bytes(wd.B, wd.H, wd.d_k, wd.d_v) - wd.B * wd.H * 4 * wd.d_k + wd.B * wd.H * 4
    out["decode"] = {"workload": "delta decode: B=256 H=32 d=128 bf16 q/k/v, fp32 beta, fp32 state, %d steps" % T,
                     "ms_per_step": dper, "tokens_per_s": wd.B / (dper / 1e3),
                     "GB_per_s": dbytes / (dper / 1e3) / 1e9,
                     "hbm_frac": dbytes / (dper / 1e3) / 1e9 / HBM_PEAK_GBS, "bytes_per_step": dbytes}
    return out


def run_gate(args, torch, api, inputs):
    """The input-side gate producer ("Gated Linear Attention", Recurrent Form:
    alpha_t = sigmoid(W_up W_down x_t)) at the gla_prefill shape: the log-gates that the
    headline prefill reads, produced from a d_model = 2048 input with rank-16 weights."""
    w = inputs.GATE_WORKLOAD
    d = inputs.draw_gate(device="cuda")
    g = torch.empty(w["B"], w["H"], w["L"], w["d_k"], dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        api.gate_project(d["x"], d["w_down"], d["w_up"], w["H"], w["d_k"], tau=w["tau"], out=g, stream=stream)

    _settle(torch, step, args.settle_s / 4)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    n = max(5, args.steps // 2)
    per = _events_ms(step, n, stream) / n
    es = 2
    ntok = w["B"] * w["L"]
    nbytes = ntok * w["d_model"] * es + (w["rank"] * w["d_model"] + w["H"] * w["d_k"] * w["rank"]) * es \
        + ntok * w["H"] * w["d_k"] * 4
    flops = 2 * ntok * w["rank"] * (w["d_model"] + w["H"] * w["d_k"])
    gbs = nbytes / (per / 1e3) / 1e9
    return {"workload": "gate_project: B=8 L=4096 d_model=2048 rank 16 -> H=16 x d_k=128 fp32 log-gates, "
                        "bf16 x and weights, tau 16",
            "ms_per_step": per, "tokens_per_s": ntok / (per / 1e3), "GB_per_s": gbs,
            "hbm_frac": gbs / HBM_PEAK_GBS, "bytes_per_launch": nbytes, "flops_per_launch": flops,
            "tflops": flops / (per / 1e3) / 1e12}


def run_outer(args, torch, api, inputs):
    """The outer-product gate ("Gated Linear Attention", Recurrent Form, G_t = alpha_t
    beta_t^T) at the gla_prefill shape with value-dim gates, and its decode step at
    the decode shape."""
    w = inputs.WORKLOADS["gla_prefill"]
    inp = inputs.draw(w, device="cuda")
    gv = inputs.draw_value_gate(w, device="cuda")
    o = torch.empty(w.B, w.H, w.L, w.d_v, dtype=w.dtype, device="cuda")
    s = torch.empty(w.B, w.H, w.d_k, w.d_v, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    out = {}
    for chunk in (32, 64):
        def step():
            api.prefill_outer(inp["q"], inp["k"], inp["v"], inp["g"], gv, chunk=chunk, out=o, final_state=s,
                              stream=stream)

        _settle(torch, step, args.settle_s / 4)
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        n = max(5, args.steps // 4)
        per = _events_ms(step, n, stream) / n
        nbytes = prefill_bytes(w.B, w.H, w.L, w.d_k, w.d_v) + w.B * w.H * w.L * w.d_v * 4
        gbs = nbytes / (per / 1e3) / 1e9
        out["prefill_chunk%d" % chunk] = {
            "workload": "outer-gate prefill: B=8 H=16 L=4096 d_k=d_v=128 chunk=%d, bf16 q/k/v, fp32 key- and "
                        "value-dim log-gates" % chunk,
            "ms_per_step": per, "tokens_per_s": w.B * w.L / (per / 1e3), "GB_per_s": gbs,
            "hbm_frac": gbs / HBM_PEAK_GBS, "bytes_per_launch": nbytes}
    del inp, gv, o, s
    wd = inputs.WORKLOADS["decode"]
    T = min(256, args.decode_steps)
    d = inputs.draw_decode(wd, steps=T, device="cuda")
    gvd = inputs.draw_value_gate(wd, B=T, H=wd.B * wd.H, L=1, device="cuda").reshape(T, wd.B, wd.H, wd.d_v)
    state = inputs.draw_state(wd.B, wd.H, wd.d_k, wd.d_v, seed=19, scale=0.1, device="cuda")
    od = torch.empty(wd.B, wd.H, wd.d_v, dtype=torch.bfloat16, device="cuda")
    it = iter(range(T))

    def dstep():
        t = next(it)
        api.decode_step_outer(d["q"][t], d["k"][t], d["v"][t], d["g"][t], gvd[t], state=state, out=od,
                              stream=stream)

    torch.cuda.synchronize()
    dper = _events_ms(dstep, T, stream) / T
    dbytes = decode_step_bytes(wd.B, wd.H, wd.d_k, wd.d_v) + wd.B * wd.H * wd.d_v * 4
    out["decode"] = {"workload": "outer-gate decode: B=256 H=32 d=128 bf16 q/k/v, fp32 gates and state, %d steps"
                                 % T, "ms_per_step": dper, "tokens_per_s": wd.B / (dper / 1e3),
                     "GB_per_s": dbytes / (dper / 1e3) / 1e9,
                     "hbm_frac": dbytes / (dper / 1e3) / 1e9 / HBM_PEAK_GBS, "bytes_per_step": dbytes}
    return out


def dataclass_replace(w, **kw):
    import dataclasses
    return dataclasses.replace(w, **kw)


def kernel_source_hash():
    """sha256 over the prefill kernel's sources: a traffic figure taken from counters
    applies only while this is unchanged."""
    h = hashlib.sha256()
    for name in PREFILL_SOURCES:
        with open(os.path.join(ROOT, "causal_gated_linear_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per prefill launch from the committed counter summary, or None when
    there is none or the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith(" "))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def run_copy_kernel(args, torch):
    """A plain device copy of known size (one elementwise kernel: read n bytes, write n
    bytes) for calibrating FETCH_SIZE / WRITE_SIZE against known traffic."""
    n = COPY_MIB * 2**20 // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup + args.steps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_kernel": "mul(src, 1.0, out=dst) fp32", "read_bytes": n * 4, "write_bytes": n * 4,
                      "launches": args.warmup + args.steps}))


def _counter_rows(d):
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        sys.exit("no counter_collection.csv under %s" % d)
    return rows


def _per_dispatch(rows, kernel_substr, counter):
    """Mean over dispatches of `counter` (KiB) for kernels whose name contains the
    substring; values of one dispatch (one row per counter instance) are summed."""
    per = {}
    for r in rows:
        if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        sys.exit("no %s rows for kernels matching %r" % (counter, kernel_substr))
    vals = list(per.values())
    return sum(vals) / len(vals), len(vals), per


def summarize_traffic(dirs, command):
    """Traffic summary of the prefill kernel: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by bytes / counter of the calibration copy kernel."""
    fdir, wdir, cfdir, cwdir = dirs
    copy_bytes = COPY_MIB * 2**20
    cf, ncf, _ = _per_dispatch(_counter_rows(cfdir), "MulFunctor", "FETCH_SIZE")
    cw, ncw, _ = _per_dispatch(_counter_rows(cwdir), "MulFunctor", "WRITE_SIZE")
    ff, nf, _ = _per_dispatch(_counter_rows(fdir), PREFILL_KERNEL, "FETCH_SIZE")
    fw, nw, _ = _per_dispatch(_counter_rows(wdir), PREFILL_KERNEL, "WRITE_SIZE")
    kf, kw = copy_bytes / cf, copy_bytes / cw          # bytes per counter unit
    fetch_b, write_b = ff * kf, fw * kw
    from causal_gated_linear_amd import inputs
    w = inputs.WORKLOADS["gla_prefill"]
    alg = prefill_bytes(w.B, w.H, w.L, w.d_k, w.d_v)
    lines = [
        "# HBM traffic of the prefill kernel, bf16 d_k=d_v=128, B=8 H=16 L=4096 chunk 64, key-dim gates",
        "# commands (run from the repository root, each a rocprofv3 --pmc pass of its own):",
    ] + ["#   " + c for c in command.split(" ;; ")] + [
        "# calibration: copy kernel reads and writes %d bytes per launch" % copy_bytes,
        "copy_FETCH_SIZE_KiB_per_dispatch: %.1f  (%d dispatches)" % (cf, ncf),
        "copy_WRITE_SIZE_KiB_per_dispatch: %.1f  (%d dispatches)" % (cw, ncw),
        "fetch_scale_bytes_per_unit: %.2f" % kf,
        "write_scale_bytes_per_unit: %.2f" % kw,
        "prefill_FETCH_SIZE_KiB_per_dispatch: %.1f  (%d dispatches)" % (ff, nf),
        "prefill_WRITE_SIZE_KiB_per_dispatch: %.1f  (%d dispatches)" % (fw, nw),
        "fetch_bytes_per_launch: %.0f" % fetch_b,
        "write_bytes_per_launch: %.0f" % write_b,
        "traffic_bytes_per_launch: %.0f" % (fetch_b + write_b),
        "algorithmic_bytes_per_launch: %d" % alg,
        "traffic_over_algorithmic: %.3f" % ((fetch_b + write_b) / alg),
        "kernel_source_sha256: %s" % kernel_source_hash(),
    ]
    os.makedirs(PROFILES, exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


TRAFFIC_ALL_FILE = os.path.join(PROFILES, "gla_kernels_bench_workloads_traffic.txt")


def summarize_traffic_all(dirs, command):
    """HBM traffic of every library kernel in a bench run: FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch, summed over counter instances) grouped by (kernel, grid), each
    scaled by bytes / counter of the calibration copy kernel."""
    fdir, wdir, cfdir, cwdir = dirs
    copy_bytes = COPY_MIB * 2**20
    cf, _, _ = _per_dispatch(_counter_rows(cfdir), "MulFunctor", "FETCH_SIZE")
    cw, _, _ = _per_dispatch(_counter_rows(cwdir), "MulFunctor", "WRITE_SIZE")
    kf, kw = copy_bytes / cf, copy_bytes / cw

    def groups(d, counter):
        per, key = {}, {}
        for r in _counter_rows(d):
            name = r["Kernel_Name"]
            if r["Counter_Name"] != counter or not (name.startswith("_ZN3gla") or "gla::" in name):
                continue
            grid = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
            key[r["Dispatch_Id"]] = (name, grid)
        out = {}
        for disp, v in per.items():
            out.setdefault(key[disp], []).append(v)
        return {k: (sum(v) / len(v), len(v)) for k, v in out.items()}

    fg, wg = groups(fdir, "FETCH_SIZE"), groups(wdir, "WRITE_SIZE")
    lines = ["# HBM traffic of the library's kernels for the bench.py workloads, per dispatch",
             "# (the workloads and their algorithmic bytes per launch are those of bench.py's JSON line:",
             "#  bytes_per_launch / bytes_per_step; the segmented prefills run two kernels)",
             "# commands (run from the repository root, each a rocprofv3 --pmc pass of its own):"] + \
            ["#   " + c for c in command.split(" ;; ")] + \
            ["# calibration: copy kernel reads and writes %d bytes per launch; fetch scale %.2f, "
             "write scale %.2f bytes per counter unit" % (copy_bytes, kf, kw), "",
             "%-8s %-6s %12s %12s %12s  %s" % ("grid", "calls", "fetch_MB", "write_MB", "total_MB", "kernel")]
    for k in sorted(set(fg) | set(wg), key=lambda k: -((fg.get(k, (0, 0))[0]) * kf + wg.get(k, (0, 0))[0] * kw)):
        f = fg.get(k, (0.0, 0))[0] * kf / 1e6
        w_ = wg.get(k, (0.0, 0))[0] * kw / 1e6
        calls = max(fg.get(k, (0, 0))[1], wg.get(k, (0, 0))[1])
        lines.append("%-8d %-6d %12.1f %12.1f %12.1f  %s" % (k[1], calls, f, w_, f + w_, _demangle(k[0])))
    os.makedirs(PROFILES, exist_ok=True)
    with open(TRAFFIC_ALL_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _demangle(name):
    import subprocess
    try:
        out = subprocess.run(["c++filt"], input=name, capture_output=True, text=True, timeout=10).stdout.strip()
        return out or name
    except (OSError, subprocess.SubprocessError):
        return name


def summarize_stats(d, command):
    """Text summary of a rocprofv3 --kernel-trace --stats run: rocprofv3's own per-kernel
    statistics for the GLA kernels, then the kernel trace grouped by (kernel, grid size),
    i.e. by workload, with the mean over all dispatches, over all but the first, and over
    the second half (the headline's timed steps come after its clock-settling launches)."""
    def find(pattern):
        files = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
        if not files:
            sys.exit("no %s under %s" % (pattern, d))
        with open(files[0]) as fh:
            return list(csv.DictReader(fh))
    stats, trace = find("*kernel_stats.csv"), find("*kernel_trace.csv")
    lines = ["# rocprofv3 kernel statistics of the library's kernels (kernel trace) for the bench.py workloads",
             "#   headline prefill: B=8 H=16 L=4096 d_k=d_v=128 chunk 64, bf16, key-dim gates (grid 256)",
             "#   decode:  B=256 H=32 d=128 bf16, fp32 state; its state comes from a 512-token prefill "
             "(prefill grid 16384)",
             "#   other prefills: linear_elu1 (4x8x2048, d=64), scalar_long (1x32x32768, segmented: state-only "
             "pass, then the full pass), fp32_single_head, and the normalised form at the headline shape",
             "#   delta rule at the headline shape, chunk 32: delta_fused_kernel (grid 256); "
             "delta decode at the decode shape",
             "#   gate producer: 8x4096 tokens, d_model 2048 -> 16 heads x 128 (grid 256, persistent: 2 blocks of 64 tokens each)",
             "#   outer-product gate at the headline shape, chunk 32 and 64 (prefill_kernel with gate 3, grid 256); its decode step",
             "# kernel names are mangled: prefill_kernel<T, d_k, chunk, value-column tile, gate, elu1, "
             "state-only, normalised>, DF16b = bf16, gate 1 = key-dim, 2 = scalar; decode_kernel<T, d_k, d_v, "
             "normalised>; delta_fused_kernel<T, d_k, chunk>; gate 3 = outer-product gate (key and value gates)",
             "# command (from the repository root, REPO = its absolute path):", "#   " + command, "",
             "## rocprofv3 stats (all dispatches, warm-up included)",
             "%-8s %14s %12s %12s %12s  %s" % ("calls", "total_ns", "avg_ns", "min_ns", "max_ns", "kernel")]
    for r in stats:
        if "gla::" in _demangle(r["Name"]) or r["Name"].startswith("_ZN3gla"):
            lines.append("%-8s %14.0f %12.0f %12.0f %12.0f  %s" % (
                r["Calls"], float(r["TotalDurationNs"]), float(r["AverageNs"]), float(r["MinNs"]),
                float(r["MaxNs"]), _demangle(r["Name"])))
    groups = {}
    for r in trace:
        if not r["Kernel_Name"].startswith("_ZN3gla") and "gla::" not in r["Kernel_Name"]:
            continue
        key = (r["Kernel_Name"], int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])))
        groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines += ["", "## kernel trace by workload (duration per dispatch, ns)",
              "%-8s %-8s %12s %12s %12s %12s  %s" % ("grid", "calls", "mean", "mean_2nd+", "mean_2nd_half",
                                                    "median", "kernel")]
    for (name, grid), ds in sorted(groups.items(), key=lambda kv: -len(kv[1])):
        rest = ds[1:] or ds
        med = sorted(ds)[len(ds) // 2]
        half = ds[len(ds) // 2:]
        lines.append("%-8d %-8d %12.0f %12.0f %12.0f %12.0f  %s" % (grid, len(ds), sum(ds) / len(ds),
                                                                 sum(rest) / len(rest), sum(half) / len(half),
                                                                 med, _demangle(name)))
    os.makedirs(PROFILES, exist_ok=True)
    with open(STATS_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _oracle_seconds(fn, budget_s):
    """Runs ``fn`` (one oracle call, returns its seconds) until ``budget_s`` has passed;
    returns (runs, seconds)."""
    reps, t = 0, 0.0
    while reps == 0 or t < budget_s:
        t += fn()
        reps += 1
    return reps, t


def cpu_baseline_prefill(w, inp, budget_s):
    """The fp64 oracle on a sample of one prefill workload's heads (the same input
    bits), about ``budget_s`` seconds; tokens/s scaled to the whole workload."""
    from oracle import oracle
    threads = oracle.default_threads()
    heads_all = [(b, h) for b in range(w.B) for h in range(w.H)]
    g = inp.get("g")

    def run(heads):
        pick = lambda t: None if t is None else t[[b for b, _ in heads], [h for _, h in heads]].unsqueeze(1).cpu()
        q, k, v, gg = pick(inp["q"]), pick(inp["k"]), pick(inp["v"]), pick(g)
        t0 = time.perf_counter()
        oracle.forward(q, k, v, g=gg, gate=w.gate, feature_map=w.feature_map, nthreads=threads)
        return time.perf_counter() - t0

    probe = heads_all[:min(threads, len(heads_all))]
    t_probe = run(probe)
    n = int(min(len(heads_all), max(len(probe), len(probe) * budget_s / max(t_probe, 1e-3))))
    n = max(len(probe), n // len(probe) * len(probe))
    heads = heads_all[:n]
    reps, t = _oracle_seconds(lambda: run(heads), budget_s)
    return {"value": reps * n * w.L / w.H / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "seconds": t, "heads_sampled": n, "heads_total": len(heads_all),
            "sample": "%d of %d heads x %d runs (L=%d, d_k=%d, d_v=%d, gate=%s, phi=%s), fp64 token recurrence; "
                      "tokens/s = B*L tokens, scaled as sampled heads / H" % (
                          n, len(heads_all), reps, w.L, w.d_k, w.d_v, w.gate, w.feature_map or "identity")}


def cpu_baseline_decode(dc, budget_s):
    """The fp64 oracle beside the decode workload: on one head of every sequence, the
    recurrence over the 512-token prompt plus the 1024 steps, minus the prompt alone:
    T(1536) - T(512) is the oracle's time for the steps; tokens/s scales it to all
    heads (one token per sequence per step)."""
    from oracle import oracle
    w, smp = dc["w"], dc["oracle_sample"]
    threads = oracle.default_threads()
    n = smp["q"].shape[0]
    T = dc["steps"]

    def run(L):
        cut = lambda x: x[:, :, :L].contiguous()
        t0 = time.perf_counter()
        oracle.forward(cut(smp["q"]), cut(smp["k"]), cut(smp["v"]), g=cut(smp["g"]), gate="keydim",
                       nthreads=threads)
        return time.perf_counter() - t0

    reps_f, t_full = _oracle_seconds(lambda: run(w.L + T), budget_s * 0.75)
    reps_p, t_pre = _oracle_seconds(lambda: run(w.L), budget_s * 0.25)
    steps_s = max(t_full / reps_f - t_pre / reps_p, 1e-9)          # the T steps on n heads
    whole = steps_s * (w.B * w.H) / n                              # the T steps on every head
    return {"value": w.B * T / whole, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "seconds": t_full + t_pre, "heads_sampled": n, "heads_total": w.B * w.H,
            "ms_per_step_all_heads": whole / T * 1e3,
            "sample": "one head of each of the %d sequences: T(%d tokens) - T(%d tokens) of the fp64 token "
                      "recurrence (%d and %d runs), scaled to all %d heads; tokens/s = sequences x steps / time"
                      % (n, w.L + T, w.L, reps_f, reps_p, w.B * w.H)}


def cpu_baseline_per_core(pf, budget_s):
    """The oracle on one thread, one head of the headline prefill: tokens/s of one
    core, counted as head-tokens (L per head)."""
    from oracle import oracle
    inp, w = pf["inp"], pf["w"]
    pick = lambda t: t[0:1, 0:1].cpu()
    q, k, v, g = pick(inp["q"]), pick(inp["k"]), pick(inp["v"]), pick(inp["g"])

    def run():
        t0 = time.perf_counter()
        oracle.forward(q, k, v, g=g, gate="keydim", nthreads=1)
        return time.perf_counter() - t0

    reps, t = _oracle_seconds(run, budget_s)
    return {"head_tokens_per_s": reps * w.L / t, "tokens_per_s_equiv": reps * w.L / w.H / t, "cores": 1,
            "runs": reps, "seconds": t,
            "sample": "one head of the headline prefill (L=%d, d=%d), one thread" % (w.L, w.d_k)}


def cpu_baseline(pf, budget_s):
    """The fp64 oracle, unchanged, on a sample of the prefill workload's heads (same
    input bits), sized to roughly ``budget_s`` seconds on this host's cores."""
    from oracle import oracle
    w, inp = pf["w"], pf["inp"]
    threads = oracle.default_threads()
    heads_all = [(b, h) for b in range(w.B) for h in range(w.H)]

    def run(heads):
        pick = lambda t: t[[b for b, _ in heads], [h for _, h in heads]].unsqueeze(1).cpu()
        q, k, v, g = pick(inp["q"]), pick(inp["k"]), pick(inp["v"]), pick(inp["g"])
        t0 = time.perf_counter()
        oracle.forward(q, k, v, g=g, gate="keydim", nthreads=threads)
        return time.perf_counter() - t0

    probe = heads_all[:threads]
    t_probe = run(probe)
    n = int(min(len(heads_all), max(len(probe), len(probe) * budget_s / max(t_probe, 1e-3))))
    n = max(threads, n // threads * threads) if n >= threads else n
    heads = heads_all[:n]
    reps, t = 0, 0.0
    while reps == 0 or t < budget_s:                     # repeat a sample that is quick
        t += run(heads)
        reps += 1
    tok_s = reps * n * w.L / w.H / t                     # full-workload tokens (B*L) per second
    return {"value": tok_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d heads of the prefill workload (L=%d, d=%d, key-dim gates) x %d runs, fp64 "
                      "token recurrence, %.1f s; tokens/s scaled as heads/H" % (n, len(heads_all), w.L,
                                                                               w.d_k, reps, t)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-s", type=float, default=2.0,
                    help="untimed launches of the headline step for at least this many seconds "
                         "before the warm-up steps, so that the GPU clocks have settled")
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true", help="skip the other prefill workloads")
    ap.add_argument("--cpu-budget-s", type=float, default=30.0,
                    help="total seconds of oracle time beside the GPU figures (split over the workloads)")
    ap.add_argument("--copy-kernel", action="store_true")
    ap.add_argument("--summarize-stats", metavar="DIR")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"))
    ap.add_argument("--summarize-traffic-all", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="per-kernel HBM traffic of a whole bench run (counter passes over bench.py)")
    ap.add_argument("--command", default="", help="profile command recorded in a summary")
    args = ap.parse_args()
    if args.summarize_stats:
        return summarize_stats(args.summarize_stats, args.command)
    if args.summarize_traffic:
        return summarize_traffic(args.summarize_traffic, args.command)
    if args.summarize_traffic_all:
        return summarize_traffic_all(args.summarize_traffic_all, args.command)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the GLA kernels here are single-GPU "
              "(heads and batch shard across GPUs with no communication; see the design "
              "notes). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from causal_gated_linear_amd import api, inputs

    torch.cuda.set_device(0)
    if args.copy_kernel:
        return run_copy_kernel(args, torch)
    pf = run_prefill(args, torch, api, inputs)
    w = pf["w"]
    per_s = pf["ms_per_step"] / 1e3
    tok_s = w.B * w.L / per_s
    achieved_gbs = pf["bytes"] / per_s / 1e9
    tflops = pf["flops"] / per_s / 1e12
    line = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"seconds": args.settle_s, "launches": pf["settle_launches"],
                   "note": "untimed headline launches before the warm-up steps (clock ramp)"},
        "launch_stats": dict(pf["launch_stats"], note="after the timed region: single launches, each "
                             "between its own events"),
        "ms_per_step": pf["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gla_prefill: B=8 H=16 L=4096 d_k=d_v=128 chunk=64, bf16 q/k/v, "
                               "fp32 key-dim log-gates, fp32 final state",
                   "B": w.B, "H": w.H, "L": w.L, "d_k": w.d_k, "d_v": w.d_v, "chunk": w.chunk,
                   "gate": "keydim"},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": stored_traffic(),
                     "kernel": "gla::prefill_kernel (bf16, d_k 128, chunk 64, key-dim gate)",
                     "bytes_per_launch": pf["bytes"]},
        "mfma": {"tflops": tflops, "peak_tflops": BF16_MFMA_PEAK_TFLOPS,
                 "frac": tflops / BF16_MFMA_PEAK_TFLOPS, "flops_per_launch": pf["flops"],
                 "count": "causal"},
    }
    if not args.no_decode:
        dc = run_decode(args, torch, api, inputs)
        dper = dc["ms_per_step"] / 1e3
        dgbs = dc["bytes"] / dper / 1e9
        line["decode"] = {"workload": "decode: B=256 H=32 d=128 fp32 state, %d steps after a 512-token "
                                      "prefill" % dc["steps"],
                          "tokens_per_s": dc["w"].B / dper, "ms_per_step": dc["ms_per_step"],
                          "ms_per_step_cold": dc["ms_per_step_cold"],
                          "GB_per_s": dgbs, "hbm_frac": dgbs / HBM_PEAK_GBS,
                          "bytes_per_step": dc["bytes"]}
        nper = dc["norm_ms_per_step"] / 1e3
        line["decode_norm"] = {"workload": "normalised decode, same shape, elu+1, %d steps" % dc["norm_steps"],
                               "tokens_per_s": dc["w"].B / nper, "ms_per_step": dc["norm_ms_per_step"],
                               "GB_per_s": dc["norm_bytes"] / nper / 1e9,
                               "hbm_frac": dc["norm_bytes"] / nper / 1e9 / HBM_PEAK_GBS,
                               "bytes_per_step": dc["norm_bytes"]}
    other_baselines = None if args.no_cpu_baseline else {}
    if not args.no_others:
        line["other_prefill"] = run_other_prefills(args, torch, api, inputs, other_baselines)
        line["delta"] = run_delta(args, torch, api, inputs)
        line["gate_producer"] = run_gate(args, torch, api, inputs)
        line["outer_gate"] = run_outer(args, torch, api, inputs)
    pk = achievable_peaks()
    hbm_ach, mfma_ach = pk["hbm_GBs"], pk["mfma_bf16_tflops"]
    line["roofline"]["achievable_peak"] = hbm_ach
    line["roofline"]["achievable_frac"] = achieved_gbs / hbm_ach if hbm_ach else None
    line["mfma"]["achievable_peak_tflops"] = mfma_ach
    line["mfma"]["achievable_frac"] = tflops / mfma_ach if mfma_ach else None
    line["achievable_peaks"] = pk
    if "decode" in line and pk.get("hbm_inplace_GBs"):
        line["decode"]["achievable_peak"] = pk["hbm_inplace_GBs"]
        line["decode"]["achievable_frac"] = line["decode"]["GB_per_s"] / pk["hbm_inplace_GBs"]
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(pf, args.cpu_budget_s * 0.5)
        per_w = {"gla_prefill": dict(line["cpu_baseline"])}
        per_w.update(other_baselines or {})
        if not args.no_decode:
            per_w["decode"] = cpu_baseline_decode(dc, args.cpu_budget_s * 0.25)
        line["cpu_baseline"]["per_workload"] = per_w
        line["cpu_baseline"]["per_core"] = cpu_baseline_per_core(pf, args.cpu_budget_s * 0.1)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
