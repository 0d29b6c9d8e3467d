"""Seeded synthetic inputs for the five gated-linear-attention workloads.

This module only draws random numbers and casts them; it holds none of the
attention arithmetic.  It serves both the HIP path and the CPU oracle: every test
draws its inputs here once and hands the very same bits to both sides.

Workload recipes (shapes and distributions as specified for the runs; the pages
use the same symbols: q, k, v, per-key-dimension log-gates, the elu+1 feature map
of the "Transformers are RNNs" notes and the Mamba2 scalar gate of "Gated Linear
Attention", section "Motivation"):

  fp32_single_head   fp32, B=1 H=1 L=256 d=16, q,k ~ N(0,1)/sqrt(d_k), v ~ N(0,1),
                     key-dim log-gate g = logsigmoid(z)/16, z ~ N(0,1), chunk 16
  linear_elu1        bf16, B=4 H=8 L=2048 d=64, q,k,v ~ N(0,1), no gate (alpha = 1),
                     phi(x) = elu(x)+1 on q and k, chunk 64
  gla_prefill        bf16, B=8 H=16 L=4096 d=128, q,k ~ N(0,1)/sqrt(d_k), v ~ N(0,1),
                     key-dim g = logsigmoid(z)/16 in fp32, chunk 64
  scalar_long        bf16, B=1 H=32 L=32768 d=128, q,k,v as gla_prefill, scalar gate
                     log(gamma) = logsigmoid(z+4) per head and token, chunk 64
  decode             B=256 H=32 d=128: a 512-token gla_prefill-style prefill fills the
                     fp32 state, then 1024 single-token steps with bf16 q,k,v and
                     key-dim gates drawn as in gla_prefill

Draw order for one call: q, k, v, z, each standard normal in fp32 on the chosen
device from ``torch.Generator(device).manual_seed(seed)``, then scaled and cast
(bf16 casts round to nearest even).

The delta rule ("Attention is recurrent", Delta attention) has its own recipe,
drawn by ``draw_delta`` / ``draw_delta_decode`` in the same order (q, k, v, z):

  delta_prefill      bf16, B=8 H=16 L=4096 d=128 (the gla_prefill shape), q and k
                     ~ N(0,1) rescaled to unit length per token (in fp32, before the
                     cast), v ~ N(0,1), write strength beta = sigmoid(z) in fp32 per
                     head and token, chunk 32

The outer-product gate (G_t = alpha_t beta_t^T, same section) reuses a workload's
q, k, v and key-dim gates and adds value-dim log-gates from ``draw_value_gate``: the
same recipe logsigmoid(z)/16, z ~ N(0,1), drawn with seed + 3571.

Strong gates.  The pages put every gate in (0, 1) with no lower bound ("Gated Linear
Attention", Recurrent Form), so the key-dim and outer-gate prefills are also checked
with log-gates far below the workloads' logsigmoid(z)/16, drawn by ``draw_strong_gate``
([B, H, L, d], fp32, from its own seed):

  tau1      logsigmoid(z), z ~ N(0,1): the page's own sigma(W_up W_down x), tau = 1
  const3    g = -3 everywhere (alpha = 0.0498)
  vanish    g = -1000 everywhere (alpha underflows to 0 even in fp64)
  mixed     half of the dimensions logsigmoid(z)/16, the other half logsigmoid(z) - 6
  bursts    logsigmoid(z)/16, with every token t = 37 (mod 53) set to -200 in every
            dimension (a reset), so that strong and weak chunks alternate

The gate producer ("Gated Linear Attention", Recurrent Form: alpha_t =
sigmoid(W_up W_down x_t)) has synthetic weights, drawn by ``draw_gate`` in the
order x, W_down, W_up:

  gate_project       bf16, B=8 L=4096 d_model=2048 (= H d_k of gla_prefill), rank 16,
                     H=16 d_k=128, x ~ N(0,1), W_down ~ N(0,1)/sqrt(d_model),
                     W_up ~ N(0,1)/sqrt(rank), tau 16: z is about N(0,1), so the
                     produced gates follow the gla_prefill recipe logsigmoid(z)/16
"""
from __future__ import annotations

import dataclasses
import math

import torch
import torch.nn.functional as F


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: torch.dtype
    B: int
    H: int
    L: int
    d_k: int
    d_v: int
    chunk: int
    gate: str | None            # None, "keydim" or "scalar"
    feature_map: str | None     # None or "elu1"
    scale_qk: bool              # q, k drawn as N(0,1)/sqrt(d_k)
    decode_steps: int = 0       # > 0 only for the decode workload
    seed: int = 0


WORKLOADS = {
    "fp32_single_head": Workload("fp32_single_head", torch.float32, 1, 1, 256, 16, 16, 16,
                                 "keydim", None, True, seed=1),
    "linear_elu1": Workload("linear_elu1", torch.bfloat16, 4, 8, 2048, 64, 64, 64,
                            None, "elu1", False, seed=2),
    "gla_prefill": Workload("gla_prefill", torch.bfloat16, 8, 16, 4096, 128, 128, 64,
                            "keydim", None, True, seed=3),
    "scalar_long": Workload("scalar_long", torch.bfloat16, 1, 32, 32768, 128, 128, 64,
                            "scalar", None, True, seed=4),
    "decode": Workload("decode", torch.bfloat16, 256, 32, 512, 128, 128, 64,
                       "keydim", None, True, decode_steps=1024, seed=5),
    "delta_prefill": Workload("delta_prefill", torch.bfloat16, 8, 16, 4096, 128, 128, 32,
                              None, None, False, seed=6),
}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _log_gate(z, gate):
    """The configured log-gate recipes (input distributions, not attention math)."""
    if gate == "keydim":
        return F.logsigmoid(z) / 16.0
    if gate == "scalar":
        return F.logsigmoid(z + 4.0)
    raise ValueError(gate)


def draw(w: Workload, *, B=None, H=None, L=None, seed=None, device="cpu"):
    """Draw q, k, v (and g) for a prefill over shape [B, H, L, d] of workload ``w``.

    Sizes default to the workload's own; tests override them to get oracle-sized
    cases of the same distributions.  Returns a dict of tensors on ``device``.
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    L = w.L if L is None else L
    seed = w.seed if seed is None else seed
    gen = _gen(device, seed)
    f32 = dict(dtype=torch.float32, device=device, generator=gen)
    qk_scale = 1.0 / math.sqrt(w.d_k) if w.scale_qk else 1.0
    q = torch.randn(B, H, L, w.d_k, **f32) * qk_scale
    k = torch.randn(B, H, L, w.d_k, **f32) * qk_scale
    v = torch.randn(B, H, L, w.d_v, **f32)
    g = None
    if w.gate == "keydim":
        g = _log_gate(torch.randn(B, H, L, w.d_k, **f32), "keydim")
    elif w.gate == "scalar":
        g = _log_gate(torch.randn(B, H, L, **f32), "scalar")
    return dict(q=q.to(w.dtype), k=k.to(w.dtype), v=v.to(w.dtype),
                g=None if g is None else g.contiguous())


def draw_decode(w: Workload, *, steps=None, B=None, H=None, seed=None, device="cpu"):
    """Draw the per-step decode inputs, step-major: q, k [T, B, H, d_k], v [T, B, H, d_v],
    g [T, B, H, d_k] (key-dim) or [T, B, H] (scalar).  Seeded apart from ``draw``."""
    T = w.decode_steps if steps is None else steps
    B = w.B if B is None else B
    H = w.H if H is None else H
    seed = (w.seed if seed is None else seed) + 7919
    gen = _gen(device, seed)
    f32 = dict(dtype=torch.float32, device=device, generator=gen)
    qk_scale = 1.0 / math.sqrt(w.d_k) if w.scale_qk else 1.0
    q = torch.randn(T, B, H, w.d_k, **f32) * qk_scale
    k = torch.randn(T, B, H, w.d_k, **f32) * qk_scale
    v = torch.randn(T, B, H, w.d_v, **f32)
    g = None
    if w.gate == "keydim":
        g = _log_gate(torch.randn(T, B, H, w.d_k, **f32), "keydim")
    elif w.gate == "scalar":
        g = _log_gate(torch.randn(T, B, H, **f32), "scalar")
    return dict(q=q.to(w.dtype), k=k.to(w.dtype), v=v.to(w.dtype),
                g=None if g is None else g.contiguous())


def draw_state(B, H, d_k, d_v, *, seed, scale=1.0, device="cpu"):
    """A random fp32 initial state [B, H, d_k, d_v] ~ scale * N(0,1)."""
    gen = _gen(device, seed)
    return torch.randn(B, H, d_k, d_v, dtype=torch.float32, device=device, generator=gen) * scale


def _unit_rows(x):
    """Rescale the last axis to unit length (an input distribution, as the gates' recipe)."""
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-6)


def draw_delta(w: Workload, *, B=None, H=None, L=None, seed=None, device="cpu"):
    """Draw q, k (unit rows), v and beta [B, H, L] for a delta-rule prefill."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    L = w.L if L is None else L
    seed = w.seed if seed is None else seed
    gen = _gen(device, seed)
    f32 = dict(dtype=torch.float32, device=device, generator=gen)
    q = _unit_rows(torch.randn(B, H, L, w.d_k, **f32))
    k = _unit_rows(torch.randn(B, H, L, w.d_k, **f32))
    v = torch.randn(B, H, L, w.d_v, **f32)
    beta = torch.sigmoid(torch.randn(B, H, L, **f32))
    return dict(q=q.to(w.dtype), k=k.to(w.dtype), v=v.to(w.dtype), beta=beta.contiguous())


def draw_delta_decode(w: Workload, *, steps, B=None, H=None, seed=None, device="cpu"):
    """Step-major delta-rule decode inputs: q, k [T, B, H, d_k], v [T, B, H, d_v],
    beta [T, B, H].  Seeded apart from ``draw_delta``."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    seed = (w.seed if seed is None else seed) + 7919
    gen = _gen(device, seed)
    f32 = dict(dtype=torch.float32, device=device, generator=gen)
    q = _unit_rows(torch.randn(steps, B, H, w.d_k, **f32))
    k = _unit_rows(torch.randn(steps, B, H, w.d_k, **f32))
    v = torch.randn(steps, B, H, w.d_v, **f32)
    beta = torch.sigmoid(torch.randn(steps, B, H, **f32))
    return dict(q=q.to(w.dtype), k=k.to(w.dtype), v=v.to(w.dtype), beta=beta.contiguous())


GATE_WORKLOAD = dict(B=8, L=4096, d_model=2048, rank=16, H=16, d_k=128, tau=16.0, dtype=torch.bfloat16, seed=7)


def draw_gate(*, B=None, L=None, d_model=None, rank=None, H=None, d_k=None, dtype=None, seed=None,
              device="cpu"):
    """Draw x [B, L, d_model], W_down [rank, d_model] and W_up [H*d_k, rank] for the
    gate producer (sizes default to GATE_WORKLOAD)."""
    w = dict(GATE_WORKLOAD)
    for k, v in dict(B=B, L=L, d_model=d_model, rank=rank, H=H, d_k=d_k, dtype=dtype, seed=seed).items():
        if v is not None:
            w[k] = v
    gen = _gen(device, w["seed"])
    f32 = dict(dtype=torch.float32, device=device, generator=gen)
    x = torch.randn(w["B"], w["L"], w["d_model"], **f32)
    wd = torch.randn(w["rank"], w["d_model"], **f32) / math.sqrt(w["d_model"])
    wu = torch.randn(w["H"] * w["d_k"], w["rank"], **f32) / math.sqrt(w["rank"])
    dt = w["dtype"]
    return dict(x=x.to(dt), w_down=wd.to(dt), w_up=wu.to(dt))


def draw_value_gate(w: Workload, *, B=None, H=None, L=None, seed=None, device="cpu"):
    """Value-dimension log-gates [B, H, L, d_v] for the outer-product gate, drawn like
    the key-dimension gates (logsigmoid(z)/16) from their own seed."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    L = w.L if L is None else L
    seed = (w.seed if seed is None else seed) + 3571
    gen = _gen(device, seed)
    z = torch.randn(B, H, L, w.d_v, dtype=torch.float32, device=device, generator=gen)
    return _log_gate(z, "keydim").contiguous()


STRONG_GATES = ("tau1", "const3", "vanish", "mixed", "bursts")


def draw_strong_gate(kind, B, H, L, d, *, seed, device="cpu"):
    """Log-gates [B, H, L, d] (fp32) of one of the STRONG_GATES recipes above."""
    gen = _gen(device, seed)
    z = torch.randn(B, H, L, d, dtype=torch.float32, device=device, generator=gen)
    if kind == "tau1":
        g = F.logsigmoid(z)
    elif kind == "const3":
        g = torch.full_like(z, -3.0)
    elif kind == "vanish":
        g = torch.full_like(z, -1000.0)
    elif kind == "mixed":
        g = torch.where(torch.arange(d, device=device) % 2 == 0, F.logsigmoid(z) / 16.0, F.logsigmoid(z) - 6.0)
    elif kind == "bursts":
        g = F.logsigmoid(z) / 16.0
        g[:, :, 37::53, :] = -200.0
    else:
        raise ValueError(kind)
    return g.contiguous()
