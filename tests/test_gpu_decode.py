"""GPU parity of gla_decode_step (through the C ABI) against the fp64 oracle: one
decode step is one token of the recurrence from the given state, so n steps from
S0 must match the oracle run over those n tokens from S0, output by output."""
import numpy as np
import pytest
import torch

from causal_gated_linear_amd import api, inputs
from oracle import oracle
from tests import util

pytestmark = pytest.mark.gpu
DEV = "cuda"
W = inputs.WORKLOADS


def _steps_vs_oracle(w, B, H, T, seed, s0_scale=0.5):
    d = inputs.draw_decode(w, steps=T, B=B, H=H, seed=seed)           # step-major [T, B, H, ...]
    s0 = inputs.draw_state(B, H, w.d_k, w.d_v, seed=seed + 1, scale=s0_scale)
    state = s0.to(DEV)
    dd = {k: (None if v is None else v.to(DEV)) for k, v in d.items()}
    outs = []
    for t in range(T):
        o = api.decode_step(dd["q"][t], dd["k"][t], dd["v"][t],
                            log_gate=None if dd["g"] is None else dd["g"][t],
                            state=state, gate=w.gate, feature_map=w.feature_map)
        outs.append(o)
    torch.cuda.synchronize()
    o_gpu = torch.stack(outs, dim=2)                                   # [B, H, T, d_v]
    seq = lambda x: None if x is None else x.movedim(0, 2).contiguous()  # -> [B, H, T, ...]
    ro, rs = oracle.forward(seq(d["q"]), seq(d["k"]), seq(d["v"]), g=seq(d["g"]), gate=w.gate,
                            feature_map=w.feature_map, s0=s0)
    tol = util.TOL[w.dtype]
    eo = util.assert_close(o_gpu, ro, tol, "%s decode o" % w.name)
    es = util.assert_close(state, rs, tol, "%s decode state" % w.name)
    print("%s decode B=%d H=%d T=%d: err o %.2e s %.2e" % (w.name, B, H, T, eo, es))


@pytest.mark.parametrize("name", ["decode", "fp32_single_head", "linear_elu1", "scalar_long"])
def test_decode_steps(name):
    _steps_vs_oracle(W[name], 3, 5, 9, seed=20 + len(name))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (128, 16), (16, 128), (64, 32)])
def test_decode_dims(dtype, dk, dv):
    w = inputs.Workload("dims", dtype, 2, 3, 0, dk, dv, 64, "keydim", "elu1", True, seed=0)
    _steps_vs_oracle(w, 2, 3, 4, seed=dk + dv)


def test_decode_with_library_allocated_state():
    """gla_state_alloc gives a zeroed state usable by decode; freed by gla_state_free."""
    w = W["decode"]
    st = api.state_alloc(2, 4, 128, 128)
    s = st.tensor()
    torch.cuda.synchronize()
    assert s.shape == (2, 4, 128, 128) and torch.count_nonzero(s).item() == 0
    d = inputs.draw_decode(w, steps=3, B=2, H=4, seed=31)
    dd = {k: v.to(DEV) for k, v in d.items()}
    outs = [api.decode_step(dd["q"][t], dd["k"][t], dd["v"][t], log_gate=dd["g"][t], state=s,
                            gate="keydim") for t in range(3)]
    torch.cuda.synchronize()
    seq = lambda x: x.movedim(0, 2).contiguous()
    ro, rs = oracle.forward(seq(d["q"]), seq(d["k"]), seq(d["v"]), g=seq(d["g"]), gate="keydim")
    util.assert_close(torch.stack(outs, 2), ro, 2e-2, "decode o (library state)")
    util.assert_close(s, rs, 2e-2, "decode state (library state)")
    del s
    st.free()


def test_prefill_then_decode_equals_longer_prefill():
    """prefill(L) followed by n decode steps equals the recurrence over L + n tokens."""
    w = W["decode"]
    B, H, L, T = 2, 3, 200, 12
    pre = inputs.draw(w, B=B, H=H, L=L, seed=41)
    d = inputs.draw_decode(w, steps=T, B=B, H=H, seed=41)
    pdev = {k: v.to(DEV) for k, v in pre.items()}
    _, state = api.prefill(pdev["q"], pdev["k"], pdev["v"], log_gate=pdev["g"], gate="keydim", chunk=64)
    dd = {k: v.to(DEV) for k, v in d.items()}
    outs = [api.decode_step(dd["q"][t], dd["k"][t], dd["v"][t], log_gate=dd["g"][t], state=state,
                            gate="keydim") for t in range(T)]
    torch.cuda.synchronize()
    cat = lambda a, b: torch.cat([a, b.movedim(0, 2)], dim=2)
    ro, rs = oracle.forward(cat(pre["q"], d["q"]), cat(pre["k"], d["k"]), cat(pre["v"], d["v"]),
                            g=cat(pre["g"], d["g"]), gate="keydim")
    util.assert_close(torch.stack(outs, 2), ro[:, :, L:], 2e-2, "decode after prefill o")
    util.assert_close(state, rs, 2e-2, "decode after prefill state")


def test_decode_full_size_one_head_per_sequence():
    """The decode workload as specified: B=256, H=32, d=128, a 512-token prefill fills
    the state, then 1024 decode steps; one head of every one of the 256 sequences is
    checked at every step's output and at the final state, against the oracle over all
    1536 tokens ("Attention is recurrent", Linear attention: each step reads only the
    cached state)."""
    w = W["decode"]
    pre = inputs.draw(w, device=DEV)
    _, state = api.prefill(pre["q"], pre["k"], pre["v"], log_gate=pre["g"], gate="keydim", chunk=w.chunk)
    d = inputs.draw_decode(w, device=DEV)
    heads = [(b, (7 * b) % w.H) for b in range(w.B)]
    bi = torch.tensor([b for b, _ in heads], device=DEV)
    hi = torch.tensor([h for _, h in heads], device=DEV)
    hist = []
    for t in range(w.decode_steps):
        o = api.decode_step(d["q"][t], d["k"][t], d["v"][t], log_gate=d["g"][t], state=state, gate="keydim")
        hist.append(o[bi, hi])
    torch.cuda.synchronize()
    o_gpu = torch.stack(hist, dim=1).unsqueeze(1)                      # [n, 1, T, d_v]
    seqs = {}
    for key in ("q", "k", "v", "g"):
        a = pre[key][bi, hi]                                           # [n, 512, d]
        bseq = d[key][:, bi, hi].transpose(0, 1)                       # [n, T, d]
        seqs[key] = torch.cat([a, bseq], dim=1).unsqueeze(1).cpu()
    ro, rs = oracle.forward(seqs["q"], seqs["k"], seqs["v"], g=seqs["g"], gate="keydim")
    eo = util.assert_close(o_gpu, ro[:, :, w.L:], 2e-2, "decode full o (every step)")
    es = util.assert_close(state[bi, hi].unsqueeze(1), rs, 2e-2, "decode full state")
    print("decode full size, one head of each of %d sequences: err o %.2e s %.2e" % (len(heads), eo, es))


def _run_steps(dd, state, t0, t1):
    return [api.decode_step(dd["q"][t], dd["k"][t], dd["v"][t], log_gate=dd["g"][t], state=state, gate="keydim")
            for t in range(t0, t1)]


def test_decode_deterministic():
    """Two runs of the same steps from the same state give the same bits (the step
    has no atomics and a fixed reduction order)."""
    w = W["decode"]
    d = inputs.draw_decode(w, steps=20, B=16, H=32, seed=51)
    dd = {k: v.to(DEV) for k, v in d.items()}
    s0 = inputs.draw_state(16, 32, w.d_k, w.d_v, seed=52, scale=0.5).to(DEV)
    a, b = s0.clone(), s0.clone()
    oa, ob = _run_steps(dd, a, 0, 20), _run_steps(dd, b, 0, 20)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(oa, ob))
    assert torch.equal(a, b)


def test_decode_checkpoint_resume_is_bitwise():
    """The state is the whole history ("Attention is recurrent", Linear attention):
    copying it to host memory after step k, restoring it into a fresh device buffer and
    continuing gives the uninterrupted run's outputs and final state, bit for bit."""
    w = W["decode"]
    T, k = 40, 17
    d = inputs.draw_decode(w, steps=T, B=8, H=32, seed=53)
    dd = {key: v.to(DEV) for key, v in d.items()}
    s0 = inputs.draw_state(8, 32, w.d_k, w.d_v, seed=54, scale=0.5).to(DEV)
    full = s0.clone()
    o_full = _run_steps(dd, full, 0, T)
    part = s0.clone()
    o_a = _run_steps(dd, part, 0, k)
    torch.cuda.synchronize()
    host = part.cpu().numpy().copy()                                   # checkpoint
    del part
    restored = torch.from_numpy(host).to(DEV)                          # resume in a new buffer
    o_b = _run_steps(dd, restored, k, T)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(o_full, o_a + o_b))
    assert torch.equal(full, restored)
