"""Shared helpers for the GPU parity tests (comparison metric, oracle calls)."""
from __future__ import annotations

import contextlib

import numpy as np
import torch

from causal_gated_linear_amd import _lib
from oracle import oracle

# Tolerances on the normwise relative error per (batch, head): max|x - ref| / max|ref|
# over that head's slice, for bf16 inputs and for fp32 inputs (fp32 accumulation).
TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}


def head_errors(x, ref):
    """Per-(b, h) normwise relative error of x against the fp64 reference.
    x, ref: [B, H, ...].  NaN/Inf anywhere in x gives inf for that head."""
    x = x.detach().to("cpu").double().numpy() if isinstance(x, torch.Tensor) else np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    B, H = ref.shape[:2]
    xf = x.reshape(B, H, -1)
    rf = ref.reshape(B, H, -1)
    err = np.zeros((B, H))
    for b in range(B):
        for h in range(H):
            if not np.all(np.isfinite(xf[b, h])):
                err[b, h] = np.inf
                continue
            den = np.max(np.abs(rf[b, h])) if rf[b, h].size else 0.0
            num = np.max(np.abs(xf[b, h] - rf[b, h])) if rf[b, h].size else 0.0
            err[b, h] = num / den if den > 0 else num
    return err


def elementwise_p99(x, ref, floor=1e-3):
    """Largest over (b, h) of the 99th percentile of the element-wise relative error
    |x - ref| / max(|ref|, floor * max|ref|) within that head: a report beside the
    normwise gate, which the floor keeps from exploding at outputs near zero."""
    x = x.detach().to("cpu").double().numpy() if isinstance(x, torch.Tensor) else np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    B, H = ref.shape[:2]
    xf, rf = x.reshape(B, H, -1), ref.reshape(B, H, -1)
    worst = 0.0
    for b in range(B):
        for h in range(H):
            if rf[b, h].size == 0:
                continue
            den = np.maximum(np.abs(rf[b, h]), floor * np.max(np.abs(rf[b, h])))
            den[den == 0] = 1.0
            e = np.abs(xf[b, h] - rf[b, h]) / den
            k = int(0.99 * (e.size - 1))
            worst = max(worst, float(np.partition(e, k)[k]))
    return worst


def assert_close(x, ref, tol, what):
    """Gate: the per-head normwise relative error (above) within tol.  Prints it beside
    the element-wise p99 report."""
    err = head_errors(x, ref)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, "%s: worst per-head error %.3e > %.1e (head %s)" % (
        what, worst, tol, np.unravel_index(np.argmax(err), err.shape) if err.size else None)
    print("%s: normwise %.2e (bound %.0e), element-wise p99 %.2e" % (what, worst, tol, elementwise_p99(x, ref)))
    return worst


def oracle_heads(inp, heads, gate, feature_map, s0=None):
    """Run the oracle on a subset of heads [(b, h), ...] of prefill inputs ``inp``
    (tensors on any device); returns (o [n,1,L,d_v], s [n,1,d_k,d_v]) stacked as a
    [n, 1, ...] batch in the order of ``heads``."""
    def pick(t):
        if t is None:
            return None
        return torch.stack([t[b, h] for b, h in heads]).unsqueeze(1).cpu()
    return oracle.forward(pick(inp["q"]), pick(inp["k"]), pick(inp["v"]), g=pick(inp.get("g")),
                          gate=gate, feature_map=feature_map, s0=pick(s0))


def pick_heads(out, heads):
    return torch.stack([out[b, h] for b, h in heads]).unsqueeze(1)


def sample_heads(B, H, n, seed=0):
    """n distinct (b, h) pairs, always including the first and the last head."""
    r = np.random.default_rng(seed)
    allh = [(b, h) for b in range(B) for h in range(H)]
    if n >= len(allh):
        return allh
    idx = set(r.choice(len(allh), size=n - 2, replace=False).tolist()) | {0, len(allh) - 1}
    while len(idx) < n:
        idx.add(int(r.integers(len(allh))))
    return [allh[i] for i in sorted(idx)]


@contextlib.contextmanager
def plan_override(prefill_tile=0, prefill_segments=0, delta_tile=0):
    """Force launch-plan choices through the library's test hook (gla_testing_set_plan)
    for the duration of the block."""
    lib = _lib.load()
    _lib.check(lib.gla_testing_set_plan(prefill_tile, prefill_segments, delta_tile), "gla_testing_set_plan")
    try:
        yield
    finally:
        lib.gla_testing_set_plan(0, 0, 0)
