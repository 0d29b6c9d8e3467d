"""The allocation-free prefill (gla_prefill_chunked_noalloc) against gla_prefill_chunked.

The allocation-free entry point runs the same kernels with the library's per-GPU
scratch array in place of the caller's workspace.  Two calls in a row on sizes that
need a workspace (few long sequences, split into segments), the second smaller, so
the second reads scratch that the first left behind: both must give the same outputs
and final states as the workspace entry point (the same kernels and plan: the same
bits), and the oracle's result within the parity bound.
"""
import pytest
import torch

from causal_gated_linear_amd import api, inputs
from oracle import oracle
from tests import util

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("name", ["gla_prefill", "scalar_long"])
def test_noalloc_matches_workspace_entry_point(name):
    w = inputs.WORKLOADS[name]
    for L, H, seed in [(64 * 70 + 13, 2, 5100), (64 * 66, 1, 5101)]:
        assert api.workspace_bytes(1, H, L, w.d_k, w.d_v, w.chunk, w.dtype) > 0
        inp = inputs.draw(w, B=1, H=H, L=L, seed=seed)
        s0 = inputs.draw_state(1, H, w.d_k, w.d_v, seed=seed + 1, scale=0.5)
        d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
        o_ref, s_ref = api.prefill(d["q"], d["k"], d["v"], log_gate=d["g"], gate=w.gate, initial_state=s0.to(DEV),
                                   chunk=w.chunk)
        o, s = api.prefill_noalloc(d["q"], d["k"], d["v"], log_gate=d["g"], gate=w.gate,
                                   initial_state=s0.to(DEV), chunk=w.chunk)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref), (name, L)
        ro, rs = oracle.forward(inp["q"], inp["k"], inp["v"], g=inp["g"], gate=w.gate, s0=s0)
        util.assert_close(o, ro, util.TOL[w.dtype], "noalloc %s L=%d o" % (name, L))
        util.assert_close(s, rs, util.TOL[w.dtype], "noalloc %s L=%d s_final" % (name, L))


def test_noalloc_unsegmented_sizes():
    """Sizes that need no workspace pass straight through (no scratch used)."""
    w = inputs.WORKLOADS["gla_prefill"]
    inp = {k: v.to(DEV) for k, v in inputs.draw(w, B=2, H=2, L=300, seed=5102).items()}
    o_ref, s_ref = api.prefill(inp["q"], inp["k"], inp["v"], log_gate=inp["g"], gate="keydim", chunk=64)
    o, s = api.prefill_noalloc(inp["q"], inp["k"], inp["v"], log_gate=inp["g"], gate="keydim", chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
