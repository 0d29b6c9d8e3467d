"""GPU parity of the key-dimension prefill under strong gates.

The pages give every gate alpha in (0, 1) with no lower bound ("Gated Linear
Attention", GLA / Recurrent Form), and a write reaches a later token scaled by the
product of the gates in between ("Attention is recurrent", Gated linear attention).
The chunk form scales keys by exp(-B) (B the cumulative log-gate inside the chunk);
chunks whose cumulative log2-gate falls below -100 run token by token instead.  These
cases drive many chunks that way, and chunks of both kinds side by side, through the
C ABI, against the fp64 oracle at the usual bounds (per-head normwise 2e-2 for bf16,
1e-4 for fp32; any NaN or Inf fails), over every head.

Gate recipes (inputs.STRONG_GATES): the page's own tau = 1 gate logsigmoid(z); g = -3;
g = -1000 (alpha = 0); half the key dimensions weak and half strong; weak gates with
a reset token every 53 tokens.
"""
import numpy as np
import pytest
import torch

from causal_gated_linear_amd import api, inputs
from oracle import gate_oracle, oracle
from tests import util

pytestmark = pytest.mark.gpu
DEV = "cuda"
KINDS = inputs.STRONG_GATES


def _draw(dtype, B, H, L, dk, dv, kind, seed, feature_map=None):
    w = inputs.Workload("strong_" + kind, dtype, B, H, L, dk, dv, 64, "keydim", feature_map, True, seed=seed)
    inp = inputs.draw(w)
    inp["g"] = inputs.draw_strong_gate(kind, B, H, L, dk, seed=seed + 17)
    return w, inp


def _dev(inp):
    return {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}


def _check(dtype, B, H, L, dk, dv, chunk, kind, seed, feature_map=None, with_s0=True):
    w, inp = _draw(dtype, B, H, L, dk, dv, kind, seed, feature_map)
    s0 = inputs.draw_state(B, H, dk, dv, seed=seed + 1, scale=0.5) if with_s0 else None
    d = _dev(inp)
    o, s = api.prefill(d["q"], d["k"], d["v"], log_gate=d["g"], gate="keydim",
                       initial_state=None if s0 is None else s0.to(DEV), chunk=chunk, feature_map=feature_map)
    torch.cuda.synchronize()
    ro, rs = oracle.forward(inp["q"], inp["k"], inp["v"], g=inp["g"], gate="keydim", feature_map=feature_map, s0=s0)
    tol = util.TOL[dtype]
    eo = util.assert_close(o, ro, tol, "%s o (chunk %d)" % (kind, chunk))
    es = util.assert_close(s, rs, tol, "%s s_final (chunk %d)" % (kind, chunk))
    print("%s %s B=%d H=%d L=%d dk=%d dv=%d chunk=%d phi=%s: err o %.2e s %.2e" % (
        kind, dtype, B, H, L, dk, dv, chunk, feature_map, eo, es))
    return o, s


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_keydim_strong_bf16(kind, chunk):
    _check(torch.bfloat16, 2, 3, 3 * chunk + 37, 128, 128, chunk, kind, seed=3000 + chunk + len(kind))


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("chunk", [16, 64])
def test_keydim_strong_fp32(kind, chunk):
    _check(torch.float32, 2, 2, 157, 64, 64, chunk, kind, seed=3100 + chunk + len(kind))


@pytest.mark.parametrize("kind", ["tau1", "vanish", "bursts"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (128, 16), (16, 128), (64, 32)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_keydim_strong_dims(kind, dk, dv, dtype):
    """Every head and value-tile width: the token-by-token chunks map their lanes
    differently for each (d_k, tile) pair."""
    _check(dtype, 2, 2, 150, dk, dv, 64, kind, seed=3200 + dk + dv + len(kind))


@pytest.mark.parametrize("kind", ["tau1", "const3", "vanish", "bursts"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_keydim_strong_elu1(kind, dtype):
    _check(dtype, 2, 2, 200, 64, 64, 64, kind, seed=3300 + len(kind), feature_map="elu1")


def test_vanishing_gate_closed_form():
    """alpha -> 0 keeps only the current write: o_t = (phi(q_t) . phi(k_t)) v_t and the
    final state is phi(k_{L-1}) v_{L-1}^T ("Attention is recurrent", Gated linear
    attention, with every gate product after the writing token equal to zero)."""
    B, H, L, d = 2, 2, 200, 128
    w, inp = _draw(torch.bfloat16, B, H, L, d, d, "vanish", seed=3400)
    dv = _dev(inp)
    o, s = api.prefill(dv["q"], dv["k"], dv["v"], log_gate=dv["g"], gate="keydim", chunk=64)
    torch.cuda.synchronize()
    q, k, v = (inp[x].double().numpy() for x in ("q", "k", "v"))
    ref_o = np.einsum("bhti,bhti->bht", q, k)[..., None] * v
    ref_s = k[:, :, -1, :, None] * v[:, :, -1, None, :]
    util.assert_close(o, ref_o, util.TOL[torch.bfloat16], "vanishing-gate o vs closed form")
    util.assert_close(s, ref_s, util.TOL[torch.bfloat16], "vanishing-gate s_final vs closed form")


@pytest.mark.parametrize("kind", ["tau1", "vanish", "bursts"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_keydim_strong_norm(kind, dtype):
    """The normalised form: the normaliser state z runs token by token beside S in the
    chunks out of range ("Transformers are RNNs" notes)."""
    B, H, L, d = 2, 2, 180, 64
    w, inp = _draw(dtype, B, H, L, d, d, kind, seed=3500 + len(kind), feature_map="elu1")
    s0 = inputs.draw_state(B, H, d, d, seed=3501, scale=0.5)
    z0 = torch.rand(B, H, d, generator=torch.Generator().manual_seed(3502)) + 0.25
    dd = _dev(inp)
    o, s, z = api.prefill_norm(dd["q"], dd["k"], dd["v"], log_gate=dd["g"], gate="keydim", initial_state=s0.to(DEV),
                               initial_norm=z0.to(DEV), chunk=64, feature_map="elu1")
    torch.cuda.synchronize()
    ro, rs, rz = oracle.forward_norm(inp["q"], inp["k"], inp["v"], g=inp["g"], gate="keydim", feature_map="elu1",
                                     s0=s0, z0=z0)
    tol = util.TOL[dtype]
    util.assert_close(o, ro, tol, "%s norm o" % kind)
    util.assert_close(s, rs, tol, "%s norm s_final" % kind)
    util.assert_close(z, rz, tol, "%s norm z_final" % kind)


@pytest.mark.parametrize("kind", ["tau1", "bursts", "const3"])
def test_keydim_strong_segmented(kind):
    """Few long sequences run as segments: the state-only pass and the full pass both
    meet chunks out of range, and the scan over segments carries gate totals far below
    the fp32 exponent range (their exponentials underflow to zero)."""
    B, H, L, d = 1, 2, 64 * 70 + 13, 128
    assert api.workspace_bytes(B, H, L, d, d, 64, torch.bfloat16) > 0
    _check(torch.bfloat16, B, H, L, d, d, 64, kind, seed=3600 + len(kind))


def test_keydim_tau1_headline_shape_all_heads():
    """The headline shape (B=8, H=16, L=4096, d=128, chunk 64) with the page's tau = 1
    gates, every head against the oracle."""
    _check(torch.bfloat16, 8, 16, 4096, 128, 128, 64, "tau1", seed=3700, with_s0=False)


def test_keydim_strong_deterministic():
    w, inp = _draw(torch.bfloat16, 2, 4, 500, 128, 128, "bursts", seed=3800)
    d = _dev(inp)
    runs = [api.prefill(d["q"], d["k"], d["v"], log_gate=d["g"], gate="keydim", chunk=64) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_gate_project_tau1_feeds_prefill(dtype):
    """The page's gate, alpha = sigmoid(W_up W_down x) at tau = 1, produced on the GPU,
    drives the key-dim prefill at chunk 64; against the oracle's gates fed to the
    oracle's recurrence."""
    B, L, H, dk = 1, 700, 2, 128
    d = inputs.draw_gate(B=B, L=L, d_model=H * dk, rank=16, H=H, d_k=dk, dtype=torch.float32, seed=3900)
    w = inputs.Workload("tau1_fed", dtype, B, H, L, dk, dk, 64, "keydim", None, True, seed=3901)
    qkv = inputs.draw(w)
    g = api.gate_project(d["x"].to(DEV), d["w_down"].to(DEV), d["w_up"].to(DEV), H, dk, tau=1.0)
    o, s = api.prefill(qkv["q"].to(DEV), qkv["k"].to(DEV), qkv["v"].to(DEV), log_gate=g, gate="keydim", chunk=64)
    torch.cuda.synchronize()
    gref = gate_oracle.gate_project(d["x"], d["w_down"], d["w_up"], H, dk, 1.0)
    # the produced chunk sums reach the token-by-token range
    sums = gref[:, :, :L // 64 * 64].reshape(B, H, -1, 64, dk).sum(axis=3)
    print("tau = 1 chunk sums of the log-gates: min %.1f, median %.1f" % (sums.min(), np.median(sums)))
    ro, rs = oracle.forward(qkv["q"], qkv["k"], qkv["v"], g=gref, gate="keydim")
    util.assert_close(o, ro, util.TOL[dtype], "tau=1 gate-fed prefill o")
    util.assert_close(s, rs, util.TOL[dtype], "tau=1 gate-fed prefill s")


# ---- the outer-product gate, G_t = alpha_t beta_t^T ("Gated Linear Attention", Recurrent Form) ----
# Its chunk form scales keys by exp(-A) and values by exp(-Bv) (key-side and value-side
# cumulative log-gates); chunks whose lowest key-side and value-side log2 totals add up
# to less than -100 run token by token.

def _check_outer(dtype, B, H, L, dk, dv, chunk, kind_k, kind_v, seed, feature_map=None):
    w, inp = _draw(dtype, B, H, L, dk, dv, kind_k, seed, feature_map)
    gv = inputs.draw_strong_gate(kind_v, B, H, L, dv, seed=seed + 29)
    s0 = inputs.draw_state(B, H, dk, dv, seed=seed + 1, scale=0.5)
    d = _dev(inp)
    o, s = api.prefill_outer(d["q"], d["k"], d["v"], d["g"], gv.to(DEV), initial_state=s0.to(DEV), chunk=chunk,
                             feature_map=feature_map)
    torch.cuda.synchronize()
    ro, rs = oracle.forward_outer(inp["q"], inp["k"], inp["v"], inp["g"], gv, feature_map=feature_map, s0=s0)
    tol = util.TOL[dtype]
    eo = util.assert_close(o, ro, tol, "outer %s/%s o (chunk %d)" % (kind_k, kind_v, chunk))
    es = util.assert_close(s, rs, tol, "outer %s/%s s_final (chunk %d)" % (kind_k, kind_v, chunk))
    print("outer %s/%s %s L=%d dk=%d dv=%d chunk=%d: err o %.2e s %.2e" % (kind_k, kind_v, dtype, L, dk, dv, chunk,
                                                                          eo, es))


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_outer_strong_both_sides(kind, chunk):
    _check_outer(torch.bfloat16, 2, 2, 3 * chunk + 37, 128, 128, chunk, kind, kind, seed=4000 + chunk + len(kind))


@pytest.mark.parametrize("kind", ["tau1", "const3", "vanish"])
@pytest.mark.parametrize("side", ["key", "value"])
def test_outer_strong_one_side(kind, side):
    """Strong gates on one side only; the other side keeps the workloads' weak recipe
    (logsigmoid(z)/16, the 'bursts' recipe without its reset tokens has no strong gate,
    so 'mixed' with its weak half is used for contrast)."""
    kk, kv = (kind, "mixed") if side == "key" else ("mixed", kind)
    _check_outer(torch.bfloat16, 2, 2, 200, 128, 64, 64, kk, kv, seed=4100 + len(kind) + len(side))


@pytest.mark.parametrize("kind", ["tau1", "vanish", "bursts"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(16, 16), (128, 32), (32, 128), (128, 128)])
def test_outer_strong_dims(kind, dtype, dk, dv):
    """fp32 with d_k = 128 and chunk 64 runs the single-role kernel, every other size
    the producer/consumer one."""
    _check_outer(dtype, 2, 2, 150, dk, dv, 64, kind, kind, seed=4200 + dk + dv + len(kind))


@pytest.mark.parametrize("kind", ["tau1", "vanish"])
def test_outer_strong_elu1(kind):
    _check_outer(torch.bfloat16, 2, 2, 170, 64, 64, 32, kind, kind, seed=4300 + len(kind), feature_map="elu1")


def test_outer_vanishing_gate_closed_form():
    """alpha, beta -> 0: o_t = (phi(q_t) . phi(k_t)) v_t."""
    B, H, L, d = 2, 2, 130, 128
    w, inp = _draw(torch.bfloat16, B, H, L, d, d, "vanish", seed=4400)
    gv = inputs.draw_strong_gate("vanish", B, H, L, d, seed=4401)
    dv = _dev(inp)
    o, s = api.prefill_outer(dv["q"], dv["k"], dv["v"], dv["g"], gv.to(DEV), chunk=64)
    torch.cuda.synchronize()
    q, k, v = (inp[x].double().numpy() for x in ("q", "k", "v"))
    ref_o = np.einsum("bhti,bhti->bht", q, k)[..., None] * v
    util.assert_close(o, ref_o, util.TOL[torch.bfloat16], "outer vanishing-gate o vs closed form")


def test_outer_tau1_headline_shape_all_heads():
    _check_outer(torch.bfloat16, 8, 16, 4096, 128, 128, 64, "tau1", "tau1", seed=4500)


# ---- the scalar gate (one log-gate per token and head, the Mamba2-style case) ----
# It takes the same factorised chunk form with one factor per row, so a chunk whose
# log2 total falls below -100 runs token by token too.

def _check_scalar(dtype, B, H, L, dk, dv, chunk, kind, seed, feature_map=None, norm=False):
    w = inputs.Workload("strong_scalar_" + kind, dtype, B, H, L, dk, dv, chunk, "scalar", feature_map, True,
                        seed=seed)
    inp = inputs.draw(w)
    inp["g"] = inputs.draw_strong_gate(kind, B, H, L, 1, seed=seed + 17)[..., 0].contiguous()
    s0 = inputs.draw_state(B, H, dk, dv, seed=seed + 1, scale=0.5)
    d = _dev(inp)
    tol = util.TOL[dtype]
    if norm:
        z0 = torch.rand(B, H, dk, generator=torch.Generator().manual_seed(seed + 2)) + 0.25
        o, s, z = api.prefill_norm(d["q"], d["k"], d["v"], log_gate=d["g"], gate="scalar", initial_state=s0.to(DEV),
                                   initial_norm=z0.to(DEV), chunk=chunk, feature_map=feature_map)
        torch.cuda.synchronize()
        ro, rs, rz = oracle.forward_norm(inp["q"], inp["k"], inp["v"], g=inp["g"], gate="scalar",
                                         feature_map=feature_map, s0=s0, z0=z0)
        util.assert_close(z, rz, tol, "scalar %s norm z_final" % kind)
    else:
        o, s = api.prefill(d["q"], d["k"], d["v"], log_gate=d["g"], gate="scalar", initial_state=s0.to(DEV),
                           chunk=chunk, feature_map=feature_map)
        torch.cuda.synchronize()
        ro, rs = oracle.forward(inp["q"], inp["k"], inp["v"], g=inp["g"], gate="scalar", feature_map=feature_map,
                                s0=s0)
    eo = util.assert_close(o, ro, tol, "scalar %s o (chunk %d)" % (kind, chunk))
    es = util.assert_close(s, rs, tol, "scalar %s s_final (chunk %d)" % (kind, chunk))
    print("scalar %s %s L=%d dk=%d dv=%d chunk=%d phi=%s norm=%s: err o %.2e s %.2e" % (
        kind, dtype, L, dk, dv, chunk, feature_map, norm, eo, es))


@pytest.mark.parametrize("kind", ["tau1", "const3", "vanish", "bursts"])
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_scalar_strong(kind, chunk, dtype):
    _check_scalar(dtype, 2, 2, 3 * chunk + 37, 64 if dtype == torch.float32 else 128, 64, chunk, kind,
                  seed=4200 + chunk + len(kind))


@pytest.mark.parametrize("kind", ["tau1", "vanish", "bursts"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (128, 16), (16, 128)])
def test_scalar_strong_dims(kind, dk, dv):
    _check_scalar(torch.bfloat16, 2, 2, 150, dk, dv, 64, kind, seed=4300 + dk + dv + len(kind))


@pytest.mark.parametrize("kind", ["tau1", "const3", "vanish"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_scalar_strong_elu1_and_norm(kind, dtype):
    _check_scalar(dtype, 2, 2, 200, 64, 64, 64, kind, seed=4400 + len(kind), feature_map="elu1")
    _check_scalar(dtype, 2, 2, 180, 64, 64, 64, kind, seed=4450 + len(kind), feature_map="elu1", norm=True)


@pytest.mark.parametrize("kind", ["tau1", "bursts", "const3"])
def test_scalar_strong_segmented(kind):
    """Few long sequences with a scalar gate are segmented; both passes meet chunks
    out of range and the scan carries totals below the fp32 range."""
    B, H, L, d = 1, 2, 64 * 70 + 13, 128
    assert api.workspace_bytes(B, H, L, d, d, 64, torch.bfloat16) > 0
    _check_scalar(torch.bfloat16, B, H, L, d, d, 64, kind, seed=4500 + len(kind))


def test_scalar_vanishing_gate_closed_form():
    """A scalar gate of 0 keeps only the current write: o_t = (q_t . k_t) v_t."""
    B, H, L, d = 2, 2, 200, 64
    w = inputs.Workload("scalar_vanish", torch.bfloat16, B, H, L, d, d, 64, "scalar", None, True, seed=4600)
    inp = inputs.draw(w)
    g = torch.full((B, H, L), -1000.0)
    dd = _dev(inp)
    o, s = api.prefill(dd["q"], dd["k"], dd["v"], log_gate=g.to(DEV), gate="scalar", chunk=64)
    torch.cuda.synchronize()
    q, k, v = (inp[x].double().numpy() for x in ("q", "k", "v"))
    util.assert_close(o, np.einsum("bhti,bhti->bht", q, k)[..., None] * v, util.TOL[torch.bfloat16],
                      "scalar vanishing-gate o vs closed form")
    util.assert_close(s, k[:, :, -1, :, None] * v[:, :, -1, None, :], util.TOL[torch.bfloat16],
                      "scalar vanishing-gate s_final vs closed form")
