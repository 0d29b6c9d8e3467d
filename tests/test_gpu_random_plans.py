"""GPU parity of the GLA prefill on seeded random combinations of the features that
select different launch plans and kernel variants, against the fp64 oracle, through
the C ABI: element type, d_k and d_v, chunk size, gate mode, feature map, batch and
head counts, lengths from one token to well past the segmentation threshold (so the
two-pass segmented plan with its state-pass pieces runs too), an initial state, and
the final state written over it in place.

The gate is the per-head normwise relative error of the other parity tests (2e-2 for
bf16, 1e-4 for fp32; NaN or Inf fails).  For sequences shorter than 16 tokens with
identity features, an output is a handful of dot products q_t . k_s that may cancel,
and the error of any evaluation with rounded gated operands is bounded relative to
the sum of the terms' magnitudes, not to the result (the usual error bound of a dot
product).  There the denominator is the oracle's output for |q|, |k|, |v| and |s0|
with the same gates, which is at least as large as the result's magnitude.
"""
import random

import numpy as np
import pytest
import torch

from causal_gated_linear_amd import api, inputs
from oracle import oracle
from tests import util

pytestmark = pytest.mark.gpu
DEV = "cuda"
CASES = 120


def _cases():
    rng = random.Random(20261203)
    out = []
    for i in range(CASES):
        dtype = rng.choice([torch.bfloat16, torch.bfloat16, torch.float32])
        dk, dv = rng.choice([16, 32, 64, 128]), rng.choice([16, 32, 64, 128])
        chunk = rng.choice([16, 32, 64] + ([128] if dk <= 64 and dtype == torch.bfloat16 else []))
        gate = rng.choice(["keydim", "scalar", None])
        fm = rng.choice([None, "elu1"])
        B, H = rng.choice([(1, 1), (1, 2), (1, 3), (2, 2), (1, 5)])
        kind = rng.random()
        if kind < 0.15:
            L = rng.choice([1, 2, 5, 15])
        elif kind < 0.75:
            L = chunk * rng.randint(1, 6) + rng.randint(0, chunk - 1)
        else:                                  # long enough to be split into segments
            L = chunk * rng.randint(64, 140) + rng.randint(0, 9)
        with_s0 = rng.random() < 0.6
        in_place = with_s0 and rng.random() < 0.5
        out.append((i, dtype, dk, dv, chunk, gate, fm, B, H, L, with_s0, in_place, rng.randint(0, 10**6)))
    return out


def _abs_errors(o, ref, ref_abs):
    """Per-head max|o - ref| / max|ref_abs|."""
    x = o.detach().cpu().double().numpy()
    B, H = ref.shape[:2]
    d = np.abs(x - ref).reshape(B, H, -1).max(axis=2)
    den = np.abs(ref_abs).reshape(B, H, -1).max(axis=2)
    bad = ~np.isfinite(x.reshape(B, H, -1)).all(axis=2)
    e = np.where(den > 0, d / np.where(den > 0, den, 1.0), d)
    return np.where(bad, np.inf, e)


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "case%d" % c[0])
def test_random_plan(case):
    i, dtype, dk, dv, chunk, gate, fm, B, H, L, with_s0, in_place, seed = case
    w = inputs.Workload("random_plan", dtype, 1, 1, 0, dk, dv, chunk, gate, fm, True, seed=0)
    inp = inputs.draw(w, B=B, H=H, L=L, seed=seed)
    s0 = inputs.draw_state(B, H, dk, dv, seed=seed + 1, scale=0.5) if with_s0 else None
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    st = None if s0 is None else s0.to(DEV)
    ws = api.workspace_bytes(B, H, L, dk, dv, chunk, dtype)
    print("case %d: %s d_k=%d d_v=%d chunk=%d gate=%s phi=%s B=%d H=%d L=%d s0=%s in place=%s workspace=%d" % (
        i, dtype, dk, dv, chunk, gate, fm, B, H, L, with_s0, in_place, ws), flush=True)
    o, s = api.prefill(d["q"], d["k"], d["v"], log_gate=d["g"], gate=gate, initial_state=st,
                       final_state=st if in_place else None, chunk=chunk, feature_map=fm)
    torch.cuda.synchronize()
    if in_place:
        assert s.data_ptr() == st.data_ptr()
    ro, rs = oracle.forward(inp["q"], inp["k"], inp["v"], g=inp["g"], gate=gate, feature_map=fm, s0=s0)
    tol = util.TOL[dtype]
    if L < 16 and fm is None:
        ab = lambda t: None if t is None else t.abs()
        ao, as_ = oracle.forward(ab(inp["q"]), ab(inp["k"]), ab(inp["v"]), g=inp["g"], gate=gate, s0=ab(s0))
        eo, es = float(_abs_errors(o, ro, ao).max()), float(_abs_errors(s, rs, as_).max())
        print("   short sequence, error against the magnitudes' sum: o %.2e s %.2e" % (eo, es))
        assert eo <= tol and es <= tol, (eo, es)
    else:
        util.assert_close(o, ro, tol, "o")
        util.assert_close(s, rs, tol, "s_final")
