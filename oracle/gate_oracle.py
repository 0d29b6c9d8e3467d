"""fp64 CPU oracle of the input-side gate producer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The product path never
does, and this module imports nothing from the product package.

"Gated Linear Attention", section "GLA / Recurrent Form" (and the flow chart under
it): the key-dimension gate of token t is alpha_t = sigmoid(W_up W_down x_t), a
low-rank map from the token's input x_t (d_model) down to r dimensions and up to
one value per key dimension of every head.  The library takes natural-log gates,
so the producer returns

    g[b, h, t, i] = log(sigmoid(z_t[h d_k + i])) / tau,   z_t = W_up (W_down x_t)

in the [B, H, L, d_k] layout of the prefill.  tau = 1 is the page's form; tau > 1
gives alpha = sigmoid(z)^(1/tau), a slower decay (the bench inputs' /16).  Inputs
are upcast exactly to float64; the two products are numpy matmuls and
log(sigmoid(z)) is written as -log(1 + e^-z) through numpy's logaddexp, which stays
finite for every z.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def gate_project(x, w_down, w_up, H, d_k, tau=1.0):
    """x: [B, L, d_model]; w_down: [r, d_model]; w_up: [H*d_k, r].  Returns the fp64
    log-gates g [B, H, L, d_k]."""
    x, w_down, w_up = _f64(x), _f64(w_down), _f64(w_up)
    B, L, dm = x.shape
    r = w_down.shape[0]
    if w_down.shape != (r, dm) or w_up.shape != (H * d_k, r):
        raise ValueError("gate oracle: shapes x %s, w_down %s, w_up %s do not fit H=%d d_k=%d"
                         % (x.shape, w_down.shape, w_up.shape, H, d_k))
    zd = x @ w_down.T                          # [B, L, r]
    z = zd @ w_up.T                            # [B, L, H*d_k]
    g = -np.logaddexp(0.0, -z) / float(tau)    # log sigmoid(z) / tau
    return np.ascontiguousarray(g.reshape(B, L, H, d_k).transpose(0, 2, 1, 3))
