"""GPU parity of the normalised form (gla_prefill_chunked_norm, gla_decode_step_norm)
against the fp64 oracle's normalised recurrence ("Transformers are RNNs" notes: the
weighted sum of values over the sum of the same weights; the normaliser state z
decays with the same gate as S).

The feature map is elu+1 throughout: its features are positive, so with z0 >= 0 every
denominator is positive.  The metric and bounds are those of the other parity tests
(per-head normwise relative error, 2e-2 bf16 / 1e-4 fp32), applied to o, the final S
and the final z.
"""
import dataclasses

import pytest
import torch

from causal_gated_linear_amd import api, inputs
from oracle import oracle
from tests import util

pytestmark = pytest.mark.gpu
DEV = "cuda"
W = inputs.WORKLOADS


def _elu1(w):
    return dataclasses.replace(w, feature_map="elu1")


def _z0(B, H, dk, seed):
    return torch.rand(B, H, dk, generator=torch.Generator().manual_seed(seed)) + 0.25


def _check(w, B, H, L, seed, chunk=None, with_init=False, in_place=False):
    inp = inputs.draw(w, B=B, H=H, L=L, seed=seed)
    s0 = inputs.draw_state(B, H, w.d_k, w.d_v, seed=seed + 1, scale=0.5) if with_init else None
    z0 = _z0(B, H, w.d_k, seed + 2) if with_init else None
    dev = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    s0d = None if s0 is None else s0.to(DEV)
    z0d = None if z0 is None else z0.to(DEV)
    o, s, z = api.prefill_norm(dev["q"], dev["k"], dev["v"], log_gate=dev["g"], gate=w.gate,
                               initial_state=s0d, initial_norm=z0d, chunk=chunk or w.chunk,
                               feature_map=w.feature_map,
                               final_state=s0d if in_place else None)
    torch.cuda.synchronize()
    if in_place:
        assert s.data_ptr() == s0d.data_ptr()
    ro, rs, rz = oracle.forward_norm(inp["q"], inp["k"], inp["v"], g=inp["g"], gate=w.gate,
                                     feature_map=w.feature_map, s0=s0, z0=z0)
    tol = util.TOL[w.dtype]
    eo = util.assert_close(o, ro, tol, "%s norm o" % w.name)
    es = util.assert_close(s, rs, tol, "%s norm s_final" % w.name)
    ez = util.assert_close(z, rz, tol, "%s norm z_final" % w.name)
    print("%s norm B=%d H=%d L=%d chunk=%s init=%s: err o %.2e s %.2e z %.2e" % (
        w.name, B, H, L, chunk or w.chunk, with_init, eo, es, ez))


SMALL = {
    "fp32_single_head": ("fp32_single_head", 2, 3, 250),
    "linear_elu1": ("linear_elu1", 2, 3, 209),
    "gla_prefill": ("gla_prefill", 2, 2, 300),
    "scalar_long": ("scalar_long", 1, 3, 1000),
}


@pytest.mark.parametrize("case", sorted(SMALL))
@pytest.mark.parametrize("with_init", [False, True])
def test_prefill_norm_small(case, with_init):
    name, B, H, L = SMALL[case]
    _check(_elu1(W[name]), B, H, L, seed=900 + len(case), with_init=with_init)


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("name", ["fp32_single_head", "gla_prefill", "scalar_long", "linear_elu1"])
def test_prefill_norm_chunk_sizes(name, chunk):
    _check(_elu1(W[name]), 1, 2, 3 * chunk + 7, seed=950 + chunk, chunk=chunk, with_init=True)


@pytest.mark.parametrize("L", [1, 15, 17, 64, 65, 129])
def test_prefill_norm_lengths(L):
    _check(_elu1(W["gla_prefill"]), 1, 2, L, seed=970 + L, with_init=True)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (128, 32), (16, 128)])
@pytest.mark.parametrize("gate", ["keydim", "scalar", None])
def test_prefill_norm_dims(dtype, dk, dv, gate):
    w = inputs.Workload("norm_dims", dtype, 1, 2, 0, dk, dv, 64, gate, "elu1", True, seed=0)
    _check(w, 1, 2, 150, seed=dk * 7 + dv, with_init=True)


def test_prefill_norm_in_place_state():
    """s_final may be s0 (each workgroup reads and writes only its own value columns)."""
    _check(_elu1(W["gla_prefill"]), 1, 2, 200, seed=990, with_init=True, in_place=True)


def test_prefill_norm_rejects_in_place_normaliser():
    """z_final may not overlap z0: every value tile of a head reads all of z0, so an
    in-place update would race between workgroups."""
    w = _elu1(W["gla_prefill"])
    inp = {k: v.to(DEV) for k, v in inputs.draw(w, B=1, H=2, L=64, seed=991).items()}
    z0 = torch.ones(1, 2, 128, device=DEV)
    with pytest.raises(api._lib.GLAError) as e:
        api.prefill_norm(inp["q"], inp["k"], inp["v"], log_gate=inp["g"], gate="keydim", initial_norm=z0,
                         final_norm=z0, feature_map="elu1")
    assert e.value.status == api._lib.GLA_ERR_ALIAS


def test_prefill_norm_long_few_heads_runs_unsegmented():
    """Sizes the plain prefill splits into segments run whole in the normalised form."""
    _check(_elu1(W["scalar_long"]), 1, 2, 64 * 70 + 3, seed=991, with_init=True)


def test_prefill_norm_full_size_all_heads():
    """The headline prefill shape (8x16x4096, d=128, key-dim gates) with elu+1 and the
    normaliser, every head against the oracle."""
    w = _elu1(W["gla_prefill"])
    inp = inputs.draw(w, device=DEV)
    o, s, z = api.prefill_norm(inp["q"], inp["k"], inp["v"], log_gate=inp["g"], gate="keydim",
                               chunk=w.chunk, feature_map="elu1")
    torch.cuda.synchronize()
    ro, rs, rz = oracle.forward_norm(inp["q"], inp["k"], inp["v"], g=inp["g"], gate="keydim", feature_map="elu1")
    tol = util.TOL[w.dtype]
    util.assert_close(o, ro, tol, "full-size norm o")
    util.assert_close(s, rs, tol, "full-size norm s_final")
    util.assert_close(z, rz, tol, "full-size norm z_final")


def _decode_vs_oracle(w, B, H, T, seed):
    d = inputs.draw_decode(w, steps=T, B=B, H=H, seed=seed)
    s0 = inputs.draw_state(B, H, w.d_k, w.d_v, seed=seed + 1, scale=0.5)
    z0 = _z0(B, H, w.d_k, seed + 2)
    state, norm = s0.to(DEV), z0.to(DEV)
    dd = {k: (None if v is None else v.to(DEV)) for k, v in d.items()}
    outs = []
    for t in range(T):
        outs.append(api.decode_step_norm(dd["q"][t], dd["k"][t], dd["v"][t],
                                         log_gate=None if dd["g"] is None else dd["g"][t], state=state,
                                         norm=norm, gate=w.gate, feature_map=w.feature_map))
    torch.cuda.synchronize()
    o_gpu = torch.stack(outs, dim=2)
    seq = lambda x: None if x is None else x.movedim(0, 2).contiguous()
    ro, rs, rz = oracle.forward_norm(seq(d["q"]), seq(d["k"]), seq(d["v"]), g=seq(d["g"]), gate=w.gate,
                                     feature_map=w.feature_map, s0=s0, z0=z0)
    tol = util.TOL[w.dtype]
    util.assert_close(o_gpu, ro, tol, "%s decode norm o" % w.name)
    util.assert_close(state, rs, tol, "%s decode norm state" % w.name)
    util.assert_close(norm, rz, tol, "%s decode norm z" % w.name)


@pytest.mark.parametrize("name", ["decode", "fp32_single_head", "linear_elu1", "scalar_long"])
def test_decode_norm_steps(name):
    _decode_vs_oracle(_elu1(W[name]), 3, 5, 9, seed=1000 + len(name))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(16, 16), (128, 16), (16, 128), (64, 32)])
def test_decode_norm_dims(dtype, dk, dv):
    w = inputs.Workload("norm_dims", dtype, 2, 3, 0, dk, dv, 64, "keydim", "elu1", True, seed=0)
    _decode_vs_oracle(w, 2, 3, 4, seed=dk + dv + 7)


def test_prefill_norm_then_decode_norm():
    """A normalised prefill's (S, z) continue in normalised decode steps exactly as the
    recurrence over the concatenated tokens."""
    w = _elu1(W["gla_prefill"])
    B, H, L, T = 1, 2, 130, 5
    inp = inputs.draw(w, B=B, H=H, L=L + T, seed=1100)
    dev = {k: v.to(DEV) for k, v in inp.items()}
    _, s, z = api.prefill_norm(dev["q"][:, :, :L].contiguous(), dev["k"][:, :, :L].contiguous(),
                               dev["v"][:, :, :L].contiguous(),
                               log_gate=dev["g"][:, :, :L].contiguous(), gate="keydim", feature_map="elu1")
    outs = []
    for t in range(L, L + T):
        outs.append(api.decode_step_norm(dev["q"][:, :, t].contiguous(), dev["k"][:, :, t].contiguous(),
                                         dev["v"][:, :, t].contiguous(), log_gate=dev["g"][:, :, t].contiguous(),
                                         state=s, norm=z, gate="keydim", feature_map="elu1"))
    torch.cuda.synchronize()
    ro, rs, rz = oracle.forward_norm(inp["q"], inp["k"], inp["v"], g=inp["g"], gate="keydim", feature_map="elu1")
    tol = util.TOL[w.dtype]
    util.assert_close(torch.stack(outs, dim=2), ro[:, :, L:], tol, "decode after prefill o")
    util.assert_close(s, rs, tol, "decode after prefill state")
    util.assert_close(z, rz, tol, "decode after prefill z")
