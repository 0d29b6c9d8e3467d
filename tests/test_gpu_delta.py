"""GPU parity of the delta rule (gla_prefill_delta, gla_decode_step_delta) against the
fp64 oracle's token recurrence ("Attention is recurrent", Delta attention:
u_t = beta_t (v_t - S_{t-1}^T k_t), S_t = S_{t-1} + k_t u_t^T, o_t = S_t^T q_t).

Inputs follow the delta_prefill recipe (unit-length q and k, beta = sigmoid of a
normal draw).  The metric and bounds are those of the other parity tests: per-head
normwise relative error, 2e-2 for bf16 inputs and 1e-4 for fp32 inputs, on o and on
the final state.
"""
import dataclasses

import pytest
import torch

from causal_gated_linear_amd import api, inputs
from oracle import oracle
from tests import util

pytestmark = pytest.mark.gpu
DEV = "cuda"
WD = inputs.WORKLOADS["delta_prefill"]


def _w(dtype=torch.bfloat16, dk=128, dv=128, chunk=32):
    return dataclasses.replace(WD, dtype=dtype, d_k=dk, d_v=dv, chunk=chunk)


def _check(w, B, H, L, seed, chunk=None, with_init=False, in_place=False):
    inp = inputs.draw_delta(w, B=B, H=H, L=L, seed=seed)
    s0 = inputs.draw_state(B, H, w.d_k, w.d_v, seed=seed + 1, scale=0.5) if with_init else None
    dev = {k: v.to(DEV) for k, v in inp.items()}
    s0d = None if s0 is None else s0.to(DEV)
    o, s = api.prefill_delta(dev["q"], dev["k"], dev["v"], dev["beta"], initial_state=s0d,
                             chunk=chunk or w.chunk, final_state=s0d if in_place else None)
    torch.cuda.synchronize()
    if in_place:
        assert s.data_ptr() == s0d.data_ptr()
    ro, rs = oracle.forward_delta(inp["q"], inp["k"], inp["v"], inp["beta"], s0=s0)
    tol = util.TOL[w.dtype]
    eo = util.assert_close(o, ro, tol, "delta o")
    es = util.assert_close(s, rs, tol, "delta s_final")
    print("delta %s dk=%d dv=%d B=%d H=%d L=%d chunk=%s init=%s: err o %.2e s %.2e" % (
        w.dtype, w.d_k, w.d_v, B, H, L, chunk or w.chunk, with_init, eo, es))


# chunks of 16 and 32 run in the fused kernel, chunks of 64 in the two-kernel path
@pytest.mark.parametrize("chunk", [32, 64])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("with_init", [False, True])
def test_prefill_delta_small(dtype, with_init, chunk):
    _check(_w(dtype, chunk=chunk), 2, 3, 250, seed=1200 + int(with_init), with_init=with_init)


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prefill_delta_chunk_sizes(dtype, chunk):
    _check(_w(dtype), 1, 2, 3 * chunk + 7, seed=1210 + chunk, chunk=chunk, with_init=True)


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("L", [1, 15, 17, 33, 64, 65, 129])
def test_prefill_delta_lengths(L, chunk):
    _check(_w(chunk=chunk), 1, 2, L, seed=1230 + L, with_init=True)


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (128, 32), (16, 128), (64, 128), (128, 16)])
def test_prefill_delta_dims(dtype, dk, dv, chunk):
    _check(_w(dtype, dk, dv, chunk), 1, 2, 150, seed=dk * 3 + dv, with_init=True)


@pytest.mark.parametrize("chunk", [32, 64])
@pytest.mark.parametrize("tile", ["16", "32", "64"])
def test_prefill_delta_value_tiles(tile, chunk):
    """Narrower value tiles per workgroup (more workgroups, idle waves) give the same result."""
    with util.plan_override(delta_tile=int(tile)):
        _check(_w(chunk=chunk), 2, 2, 200, seed=1250 + int(tile), with_init=True)


@pytest.mark.parametrize("chunk", [32, 64])
def test_prefill_delta_in_place_state(chunk):
    _check(_w(chunk=chunk), 1, 2, 200, seed=1260, with_init=True, in_place=True)


def test_prefill_delta_empty_copies_state():
    w = _w()
    s0 = inputs.draw_state(1, 2, 128, 128, seed=1261).to(DEV)
    q = torch.empty(1, 2, 0, 128, dtype=w.dtype, device=DEV)
    beta = torch.empty(1, 2, 0, dtype=torch.float32, device=DEV)
    o, s = api.prefill_delta(q, q, q, beta, initial_state=s0)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 0, 128) and torch.equal(s, s0)


def test_prefill_delta_zero_strength_keeps_state():
    """beta = 0 writes nothing: the final state is the initial one and o = S0^T q."""
    w = _w(torch.float32, 64, 32)
    inp = inputs.draw_delta(w, B=1, H=2, L=100, seed=1262)
    s0 = inputs.draw_state(1, 2, 64, 32, seed=1263)
    dev = {k: v.to(DEV) for k, v in inp.items()}
    o, s = api.prefill_delta(dev["q"], dev["k"], dev["v"], torch.zeros_like(dev["beta"]),
                             initial_state=s0.to(DEV))
    torch.cuda.synchronize()
    util.assert_close(s, s0.numpy(), 1e-6, "beta=0 state")
    util.assert_close(o, torch.einsum("bhli,bhij->bhlj", inp["q"].double(), s0.double()).numpy(), 1e-5,
                      "beta=0 output")


@pytest.mark.parametrize("chunk", [32, 64])
def test_prefill_delta_full_size_all_heads(chunk):
    """The delta_prefill shape (8x16x4096, d=128; chunk 32 is the launch configuration
    the benchmark times), every head against the oracle."""
    w = dataclasses.replace(WD, chunk=chunk)
    inp = inputs.draw_delta(w, device=DEV)
    o, s = api.prefill_delta(inp["q"], inp["k"], inp["v"], inp["beta"], chunk=w.chunk)
    torch.cuda.synchronize()
    ro, rs = oracle.forward_delta(inp["q"], inp["k"], inp["v"], inp["beta"])
    tol = util.TOL[w.dtype]
    util.assert_close(o, ro, tol, "full-size delta o")
    util.assert_close(s, rs, tol, "full-size delta s_final")


def _decode_vs_oracle(w, B, H, T, seed):
    d = inputs.draw_delta_decode(w, steps=T, B=B, H=H, seed=seed)
    s0 = inputs.draw_state(B, H, w.d_k, w.d_v, seed=seed + 1, scale=0.5)
    state = s0.to(DEV)
    dd = {k: v.to(DEV) for k, v in d.items()}
    outs = [api.decode_step_delta(dd["q"][t], dd["k"][t], dd["v"][t], dd["beta"][t], state=state)
            for t in range(T)]
    torch.cuda.synchronize()
    seq = lambda x: x.movedim(0, 2).contiguous()
    ro, rs = oracle.forward_delta(seq(d["q"]), seq(d["k"]), seq(d["v"]), seq(d["beta"]), s0=s0)
    tol = util.TOL[w.dtype]
    util.assert_close(torch.stack(outs, dim=2), ro, tol, "delta decode o")
    util.assert_close(state, rs, tol, "delta decode state")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(16, 16), (128, 16), (16, 128), (64, 32), (128, 128)])
def test_decode_delta_steps(dtype, dk, dv):
    _decode_vs_oracle(_w(dtype, dk, dv), 2, 3, 7, seed=1300 + dk + dv)


def test_prefill_delta_then_decode():
    """A delta prefill's final state continues in delta decode steps exactly as the
    recurrence over the concatenated tokens."""
    w = _w()
    B, H, L, T = 1, 2, 130, 5
    inp = inputs.draw_delta(w, B=B, H=H, L=L + T, seed=1400)
    dev = {k: v.to(DEV) for k, v in inp.items()}
    head = lambda x: x[:, :, :L].contiguous()
    _, s = api.prefill_delta(head(dev["q"]), head(dev["k"]), head(dev["v"]), head(dev["beta"]))
    outs = [api.decode_step_delta(dev["q"][:, :, t].contiguous(), dev["k"][:, :, t].contiguous(),
                                  dev["v"][:, :, t].contiguous(), dev["beta"][:, :, t].contiguous(), state=s)
            for t in range(L, L + T)]
    torch.cuda.synchronize()
    ro, rs = oracle.forward_delta(inp["q"], inp["k"], inp["v"], inp["beta"])
    tol = util.TOL[w.dtype]
    util.assert_close(torch.stack(outs, dim=2), ro[:, :, L:], tol, "decode after delta prefill o")
    util.assert_close(s, rs, tol, "decode after delta prefill state")
