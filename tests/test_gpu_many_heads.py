"""GPU parity with many heads and short sequences: grids of several workgroups per
compute unit, with the XCD-aware workgroup order active (B*H*tiles a multiple of 8)
and not (an odd head count), for the key-dim prefill, the delta rule and the
outer-product gate.  Checked on sampled heads against the fp64 oracle, with the
bounds of the other parity tests."""
import dataclasses

import pytest
import torch

from causal_gated_linear_amd import api, inputs
from oracle import oracle
from tests import util

pytestmark = pytest.mark.gpu
DEV = "cuda"
SHAPES = [(16, 20, 70), (5, 7, 33)]          # B*H = 320 (remap on) and 35 (remap off)


def _pick(t, heads):
    return torch.stack([t[b, h] for b, h in heads]).unsqueeze(1).cpu()


@pytest.mark.parametrize("B,H,L", SHAPES)
def test_keydim_prefill_many_heads(B, H, L):
    w = inputs.WORKLOADS["gla_prefill"]
    inp = inputs.draw(w, B=B, H=H, L=L, seed=1800 + B, device=DEV)
    o, s = api.prefill(inp["q"], inp["k"], inp["v"], log_gate=inp["g"], gate="keydim", chunk=64)
    torch.cuda.synchronize()
    heads = util.sample_heads(B, H, 6, seed=B + H)
    ro, rs = oracle.forward(_pick(inp["q"], heads), _pick(inp["k"], heads), _pick(inp["v"], heads),
                            g=_pick(inp["g"], heads), gate="keydim")
    util.assert_close(util.pick_heads(o, heads), ro, util.TOL[w.dtype], "many-heads o")
    util.assert_close(util.pick_heads(s, heads), rs, util.TOL[w.dtype], "many-heads s")


@pytest.mark.parametrize("chunk", [32, 64])
@pytest.mark.parametrize("B,H,L", SHAPES)
def test_delta_many_heads(B, H, L, chunk):
    w = dataclasses.replace(inputs.WORKLOADS["delta_prefill"], chunk=chunk)
    inp = inputs.draw_delta(w, B=B, H=H, L=L, seed=1850 + B, device=DEV)
    o, s = api.prefill_delta(inp["q"], inp["k"], inp["v"], inp["beta"], chunk=chunk)
    torch.cuda.synchronize()
    heads = util.sample_heads(B, H, 6, seed=B * H)
    ro, rs = oracle.forward_delta(_pick(inp["q"], heads), _pick(inp["k"], heads), _pick(inp["v"], heads),
                                  _pick(inp["beta"], heads))
    util.assert_close(util.pick_heads(o, heads), ro, util.TOL[w.dtype], "many-heads delta o")
    util.assert_close(util.pick_heads(s, heads), rs, util.TOL[w.dtype], "many-heads delta s")


@pytest.mark.parametrize("B,H,L", SHAPES)
def test_outer_many_heads(B, H, L):
    w = inputs.WORKLOADS["gla_prefill"]
    inp = inputs.draw(w, B=B, H=H, L=L, seed=1900 + B, device=DEV)
    gv = inputs.draw_value_gate(w, B=B, H=H, L=L, seed=1900 + B, device=DEV)
    o, s = api.prefill_outer(inp["q"], inp["k"], inp["v"], inp["g"], gv, chunk=32)
    torch.cuda.synchronize()
    heads = util.sample_heads(B, H, 6, seed=B + 2 * H)
    ro, rs = oracle.forward_outer(_pick(inp["q"], heads), _pick(inp["k"], heads), _pick(inp["v"], heads),
                                  _pick(inp["g"], heads), _pick(gv, heads))
    util.assert_close(util.pick_heads(o, heads), ro, util.TOL[w.dtype], "many-heads outer o")
    util.assert_close(util.pick_heads(s, heads), rs, util.TOL[w.dtype], "many-heads outer s")
