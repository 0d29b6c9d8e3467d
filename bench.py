"""Benchmark of the GLA forward on one MI355X.

One step = one chunked prefill (gla_prefill_chunked) of the headline workload:
B=8, H=16, L=4096, d_k=d_v=128, chunk 64, bf16 q/k/v, fp32 key-dimension log-gates,
final fp32 state written.  Inputs are drawn once (seeded, synthetic) and are resident
in HBM before the timed region.  The same run also times the recurrent decode
workload (B=256, H=32, d=128: a 512-token prefill fills the state, then 1024
gla_decode_step calls), and the fp64 CPU oracle on a bounded sample of the prefill
workload.

Prints ONE JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
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

METRIC = "GLA prefill tokens/s + % MFMA peak (L=4096,d=128); decode tok/s + HBM GB/s"
HBM_PEAK_GBS = 8000.0                 # MI355X HBM3E, GB/s (datasheet)
BF16_MFMA_PEAK_TFLOPS = 2516.6        # dense bf16 MFMA, TFLOP/s (256 CU x 4096 flop/clk x 2.4 GHz)


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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = _events_ms(step, args.steps, stream)          # the kernel runs on this stream
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = ms / args.steps
    nbytes = prefill_bytes(w.B, w.H, w.L, w.d_k, w.d_v)
    flops = prefill_flops(w.B, w.H, w.L, w.d_k, w.d_v, w.chunk)
    return dict(w=w, inp=inp, ms_per_step=per, wall_s=wall, bytes=nbytes, flops=flops)


def run_decode(args, torch, api, inputs):
    w = inputs.WORKLOADS["decode"]
    pre = inputs.draw(w, device="cuda")
    _, state = api.prefill(pre["q"], pre["k"], pre["v"], log_gate=pre["g"], gate="keydim", chunk=w.chunk)
    del pre
    T = args.decode_steps
    d = inputs.draw_decode(w, steps=T, device="cuda")
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
    nbytes = decode_step_bytes(w.B, w.H, w.d_k, w.d_v)
    return dict(w=w, steps=T, ms_per_step=per, bytes=nbytes)


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
    t = run(heads)
    tok_s = n * w.L / w.H / t                            # full-workload tokens (B*L) per second
    return {"value": tok_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d heads of the prefill workload (L=%d, d=%d, key-dim gates), fp64 "
                      "token recurrence, %.1f s; tokens/s scaled as heads/H" % (n, len(heads_all), w.L,
                                                                               w.d_k, t)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the GLA kernels here are single-GPU "
              "(heads and batch shard across GPUs with no communication; see the design "
              "notes). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from causal_gated_linear_amd import api, inputs

    torch.cuda.set_device(0)
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
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "gla::prefill_kernel<bf16,128,64,4>",
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
                          "GB_per_s": dgbs, "hbm_frac": dgbs / HBM_PEAK_GBS,
                          "bytes_per_step": dc["bytes"]}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(pf, args.cpu_budget_s)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
