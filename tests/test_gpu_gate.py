"""GPU parity of the input-side gate producer (gla_gate_project) against its fp64
oracle ("Gated Linear Attention", Recurrent Form: alpha_t = sigmoid(W_up W_down x_t),
written as log-gates / tau in the prefill layout).

Metric and bounds as the other parity tests: per-head normwise relative error of g,
2e-2 for bf16 inputs and 1e-4 for fp32 inputs.
"""
import numpy as np
import pytest
import torch

from causal_gated_linear_amd import api, inputs
from oracle import gate_oracle, oracle
from tests import util

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check(B, L, dm, rank, H, dk, dtype, tau, seed):
    d = inputs.draw_gate(B=B, L=L, d_model=dm, rank=rank, H=H, d_k=dk, dtype=dtype, seed=seed)
    g = api.gate_project(d["x"].to(DEV), d["w_down"].to(DEV), d["w_up"].to(DEV), H, dk, tau=tau)
    torch.cuda.synchronize()
    ref = gate_oracle.gate_project(d["x"], d["w_down"], d["w_up"], H, dk, tau)
    err = util.assert_close(g, ref, util.TOL[dtype], "gate g")
    print("gate B=%d L=%d d_model=%d rank=%d H=%d d_k=%d %s tau=%g: err %.2e" % (B, L, dm, rank, H, dk, dtype,
                                                                                  tau, err))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rank", [16, 32])
@pytest.mark.parametrize("tau", [1.0, 16.0])
def test_gate_small(dtype, rank, tau):
    _check(2, 37, 96, rank, 3, 32, dtype, tau, seed=1500 + rank)


@pytest.mark.parametrize("dk", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_gate_head_dims(dk, dtype):
    _check(1, 70, 64, 16, 2, dk, dtype, 1.0, seed=1520 + dk)


@pytest.mark.parametrize("H,dk", [(17, 128), (137, 16)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rank", [16, 32])
def test_gate_output_groups(H, dk, dtype, rank):
    """More 16-output tiles than one workgroup stages of W_up (64 KB: 128 tiles for
    bf16 rank 16, 64 for bf16 rank 32 and fp32 rank 16, 32 for fp32 rank 32), with a
    partial last group: 136 tiles, or 137 tiles of d_k = 16 whose last one is unpaired."""
    _check(2, 70, 64, rank, H, dk, dtype, 16.0, seed=1580 + H + rank)


@pytest.mark.parametrize("B,L", [(1, 1), (3, 1), (1, 64), (2, 64), (1, 65), (5, 13)])
def test_gate_token_counts(B, L):
    """Token counts below, at and across the 64-token workgroup, and workgroups that
    span a batch boundary."""
    _check(B, L, 32, 16, 2, 16, torch.bfloat16, 1.0, seed=1540 + 7 * B + L)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_gate_blocks_per_workgroup(dtype):
    """More 64-token blocks than workgroups: 601 blocks (the last one 17 tokens) over
    256 persistent workgroups, so some carry 3 blocks and reuse their first code
    buffer; every token is checked."""
    _check(1, 64 * 600 + 17, 32, 16, 1, 16, dtype, 16.0, seed=1600)


def test_gate_empty():
    d = inputs.draw_gate(B=2, L=1, d_model=32, rank=16, H=2, d_k=16, seed=1560)
    x = torch.empty(2, 0, 32, dtype=torch.bfloat16, device=DEV)
    g = api.gate_project(x, d["w_down"].to(DEV), d["w_up"].to(DEV), 2, 16)
    torch.cuda.synchronize()
    assert g.shape == (2, 2, 0, 16)


def test_gate_full_size_sampled_tokens():
    """The bench shape (B=8, L=4096, d_model=2048, rank 16, H=16, d_k=128, tau 16),
    checked on sampled tokens of every batch."""
    w = inputs.GATE_WORKLOAD
    d = inputs.draw_gate(device=DEV)
    g = api.gate_project(d["x"], d["w_down"], d["w_up"], w["H"], w["d_k"], tau=w["tau"])
    torch.cuda.synchronize()
    pos = np.sort(np.random.default_rng(3).choice(w["L"], size=48, replace=False))
    pos = np.unique(np.concatenate([pos, [0, w["L"] - 1]]))
    ref = gate_oracle.gate_project(d["x"][:, pos].cpu(), d["w_down"].cpu(), d["w_up"].cpu(), w["H"], w["d_k"],
                                   w["tau"])
    util.assert_close(g[:, :, pos], ref, util.TOL[torch.bfloat16], "full-size gate g")


def test_gate_feeds_prefill():
    """Produced gates drive the key-dim prefill: GPU gates -> GPU prefill matches the
    oracle gates -> oracle recurrence."""
    B, L, H, dk = 1, 150, 2, 64
    d = inputs.draw_gate(B=B, L=L, d_model=H * dk, rank=16, H=H, d_k=dk, dtype=torch.float32, seed=1570)
    w = inputs.Workload("gate_fed", torch.float32, B, H, L, dk, dk, 32, "keydim", None, True, seed=1571)
    qkv = inputs.draw(w)
    g = api.gate_project(d["x"].to(DEV), d["w_down"].to(DEV), d["w_up"].to(DEV), H, dk, tau=16.0)
    o, s = api.prefill(qkv["q"].to(DEV), qkv["k"].to(DEV), qkv["v"].to(DEV), log_gate=g, gate="keydim", chunk=32)
    torch.cuda.synchronize()
    gref = gate_oracle.gate_project(d["x"], d["w_down"], d["w_up"], H, dk, 16.0)
    ro, rs = oracle.forward(qkv["q"], qkv["k"], qkv["v"], g=gref, gate="keydim")
    util.assert_close(o, ro, util.TOL[torch.float32], "gate-fed prefill o")
    util.assert_close(s, rs, util.TOL[torch.float32], "gate-fed prefill s")
