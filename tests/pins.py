"""Independent forms that pin the fp64 oracle to what the pages fix.

Each ``pin_*`` function takes an oracle ``forward`` callable (the committed one, or
a deliberately broken build in the mutant tests) and returns the worst error it
found against a form of the computation that is *not* the token recurrence:

- the quadratic masked form ``(phi(Q) phi(K)^T (.) L) V`` for alpha = 1
  ("Attention is recurrent", note on non-causal linear attention: the causal case
  needs the multiplicative 0/1 mask L; "Transformers are RNNs" notes: the numerator
  as entry (i, m) of (A B^T) V with A = phi(Q), B = phi(K));
- the cumulative-sum state and the last-token regrouping Q (K^T V) ("Attention is
  recurrent", Prefill: the prefix states are a cumulative sum; note on non-causal
  linear attention: O = Q (K^T V));
- the unrolled gated form, where a write at position i reaches position n scaled
  by the product of the gates after it ("Attention is recurrent", Gated linear
  attention), evaluated with explicit products;
- exact rational arithmetic for tiny cases;
- the RetNet constant decay as a geometric mask and the Mamba2 scalar gate as the
  key-dimension gate with equal entries ("Gated Linear Attention", Motivation and
  Recurrent Form);
- closed forms: elu(x)+1 at fixed points, geometric series, vanishing gates.

Numpy and ``fractions`` only; nothing here calls the HIP path.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np


def rel_err(x, ref):
    """Normwise relative error max|x - ref| / max|ref| over the whole array."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(x - ref)) if ref.size else 0.0
    return float(num / den) if den > 0 else float(num)


def _phi(x, fm):
    if fm == "elu1":
        return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))
    return x


def rng_inputs(seed, B, H, L, dk, dv, gate=None, s0=False, g_scale=0.3):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, L, dk))
    k = r.standard_normal((B, H, L, dk))
    v = r.standard_normal((B, H, L, dv))
    g = None
    if gate == "keydim":
        g = -g_scale * r.random((B, H, L, dk))
    elif gate == "scalar":
        g = -g_scale * r.random((B, H, L))
    S0 = r.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, g, S0


# --------------------------------------------------------------------------------------
def pin_feature_map_points(fwd):
    """elu(x)+1 at x = -2, 0, 3 is e^-2, 1, 4.  With k = 0 (phi(0) = 1), v = 1 and one
    token, o_0 = phi(q)."""
    xs = np.array([-2.0, 0.0, 3.0])
    want = np.array([math.exp(-2.0), 1.0, 4.0])
    q = xs.reshape(1, 3, 1, 1)
    k = np.zeros((1, 3, 1, 1))
    v = np.ones((1, 3, 1, 1))
    o, _ = fwd(q, k, v, feature_map="elu1")
    return float(np.max(np.abs(o.reshape(3) - want)))


def pin_quadratic_masked(fwd, seed=0, fm=None, B=2, H=3, L=37, dk=5, dv=7):
    """alpha = 1: O equals (phi(Q) phi(K)^T (.) L) V per head, L_ts = [s <= t]."""
    q, k, v, _, _ = rng_inputs(seed, B, H, L, dk, dv)
    o, _ = fwd(q, k, v, feature_map=fm)
    mask = np.tril(np.ones((L, L)))
    worst = 0.0
    for b in range(B):
        for h in range(H):
            A = _phi(q[b, h], fm)
            Bm = _phi(k[b, h], fm)
            ref = ((A @ Bm.T) * mask) @ v[b, h]
            worst = max(worst, rel_err(o[b, h], ref))
    return worst


def pin_cumsum_and_last_token(fwd, seed=1, fm=None, B=2, H=2, L=29, dk=6, dv=4):
    """alpha = 1, S0 = 0: the final state is phi(K)^T V (a cumulative sum over all
    tokens), and the last output equals phi(q_last)^T (phi(K)^T V), the non-causal
    regrouping Q (K^T V) evaluated on the row that sees every token."""
    q, k, v, _, _ = rng_inputs(seed, B, H, L, dk, dv)
    o, s = fwd(q, k, v, feature_map=fm)
    worst = 0.0
    for b in range(B):
        for h in range(H):
            KV = _phi(k[b, h], fm).T @ v[b, h]
            worst = max(worst, rel_err(s[b, h], KV))
            worst = max(worst, rel_err(o[b, h, L - 1], _phi(q[b, h, L - 1], fm) @ KV))
    return worst


def unrolled_reference(q, k, v, g, gate, S0):
    """o_n = sum_{i<=n} (q_n . (k_i (.) prod_{m=i+1..n} alpha_m)) v_i
             + q_n^T Diag(prod_{m=0..n} alpha_m) S0, with explicit products."""
    B, H, L, dk = q.shape
    out = np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            if gate == "keydim":
                alpha = np.exp(g[b, h])                          # [L, dk]
            elif gate == "scalar":
                alpha = np.repeat(np.exp(g[b, h])[:, None], dk, axis=1)
            else:
                alpha = np.ones((L, dk))
            for n in range(L):
                acc = np.zeros(v.shape[3])
                for i in range(n + 1):
                    w = np.prod(alpha[i + 1:n + 1], axis=0)      # empty product = 1
                    acc += np.dot(q[b, h, n], k[b, h, i] * w) * v[b, h, i]
                if S0 is not None:
                    w0 = np.prod(alpha[0:n + 1], axis=0)
                    acc += (q[b, h, n] * w0) @ S0[b, h]
                out[b, h, n] = acc
    return out


def pin_unrolled(fwd, seed=2, gate="keydim", with_s0=True, B=2, H=2, L=23, dk=5, dv=3):
    q, k, v, g, S0 = rng_inputs(seed, B, H, L, dk, dv, gate=gate, s0=with_s0)
    o, _ = fwd(q, k, v, g=g, gate=gate, s0=S0)
    return rel_err(o, unrolled_reference(q, k, v, g, gate, S0))


def pin_exact_rational(fwd, seed=3):
    """Tiny case (L=5, d_k=3, d_v=2, B=H=1) in exact rationals via the unrolled form
    (outputs) and the expanded state sum (final state); the oracle must agree to
    ~1e-15 relative (the gates reach it as log values, exp(log a) = a + O(ulp))."""
    r = np.random.default_rng(seed)
    L, dk, dv = 5, 3, 2
    qi = r.integers(-3, 4, size=(L, dk))
    ki = r.integers(-3, 4, size=(L, dk))
    vi = r.integers(-3, 4, size=(L, dv))
    ai = r.integers(1, 8, size=(L, dk))
    a = [[Fraction(int(x), 8) for x in row] for row in ai]          # alpha in (0, 1)
    s0i = r.integers(-2, 3, size=(dk, dv))
    O = [[Fraction(0)] * dv for _ in range(L)]
    for n in range(L):
        for j in range(dv):
            tot = Fraction(0)
            for i in range(n + 1):
                for c in range(dk):
                    w = Fraction(1)
                    for m in range(i + 1, n + 1):
                        w *= a[m][c]
                    tot += int(qi[n, c]) * int(ki[i, c]) * w * int(vi[i, j])
            for c in range(dk):
                w0 = Fraction(1)
                for m in range(0, n + 1):
                    w0 *= a[m][c]
                tot += int(qi[n, c]) * w0 * int(s0i[c, j])
            O[n][j] = tot
    Sx = [[Fraction(0)] * dv for _ in range(dk)]
    for c in range(dk):
        for j in range(dv):
            w0 = Fraction(1)
            for m in range(L):
                w0 *= a[m][c]
            tot = w0 * int(s0i[c, j])
            for i in range(L):
                w = Fraction(1)
                for m in range(i + 1, L):
                    w *= a[m][c]
                tot += int(ki[i, c]) * w * int(vi[i, j])
            Sx[c][j] = tot
    g = np.log(ai / 8.0).reshape(1, 1, L, dk)
    o, s = fwd(qi.reshape(1, 1, L, dk).astype(float), ki.reshape(1, 1, L, dk).astype(float),
               vi.reshape(1, 1, L, dv).astype(float), g=g, gate="keydim",
               s0=s0i.reshape(1, 1, dk, dv).astype(float))
    O_ex = np.array([[float(x) for x in row] for row in O])
    S_ex = np.array([[float(x) for x in row] for row in Sx])
    return max(rel_err(o[0, 0], O_ex), rel_err(s[0, 0], S_ex))


def pin_scalar_is_broadcast_keydim(fwd, seed=4, B=2, H=3, L=31, dk=4, dv=5):
    """The Mamba2 gate gamma_t 1 1^T equals the key-dim gate with all entries gamma_t."""
    q, k, v, g, S0 = rng_inputs(seed, B, H, L, dk, dv, gate="scalar", s0=True)
    o1, s1 = fwd(q, k, v, g=g, gate="scalar", s0=S0)
    gk = np.repeat(g[..., None], dk, axis=3)
    o2, s2 = fwd(q, k, v, g=gk, gate="keydim", s0=S0)
    # the two must also differ from the ungated run, or the gate was ignored
    o3, _ = fwd(q, k, v, s0=S0)
    assert rel_err(o3, o2) > 1e-3
    return max(rel_err(o1, o2), rel_err(s1, s2))


def pin_retnet_geometric(fwd, seed=5, gamma=0.9, B=1, H=2, L=33, dk=4, dv=6):
    """Constant gamma (RetNet's fixed decay): O = ((Q K^T) (.) D) V with D_ts = gamma^(t-s)
    for s <= t, else 0."""
    q, k, v, _, _ = rng_inputs(seed, B, H, L, dk, dv)
    g = np.full((B, H, L), math.log(gamma))
    o, _ = fwd(q, k, v, g=g, gate="scalar")
    t = np.arange(L)
    D = np.where(t[:, None] >= t[None, :], gamma ** (t[:, None] - t[None, :]).clip(min=0), 0.0)
    worst = 0.0
    for b in range(B):
        for h in range(H):
            ref = ((q[b, h] @ k[b, h].T) * D) @ v[b, h]
            worst = max(worst, rel_err(o[b, h], ref))
    return worst


def pin_vanishing_gate(fwd, seed=6, B=1, H=2, L=9, dk=3, dv=4):
    """alpha -> 0 (g = -1000, exp underflows to 0): the state keeps only the current
    write, so o_t = (q_t . k_t) v_t and S_final = k_last v_last^T."""
    q, k, v, _, S0 = rng_inputs(seed, B, H, L, dk, dv, s0=True)
    g = np.full((B, H, L, dk), -1000.0)
    o, s = fwd(q, k, v, g=g, gate="keydim", s0=S0)
    ref = np.einsum("bhtc,bhtc->bht", q, k)[..., None] * v
    sref = np.einsum("bhc,bhj->bhcj", k[:, :, -1], v[:, :, -1])
    return max(rel_err(o, ref), rel_err(s, sref))


def pin_geometric_closed_form(fwd, alpha=0.75, s0=2.5, L=12):
    """d_k = d_v = 1, q = k = v = 1, constant alpha, initial state s0:
    o_t = alpha^(t+1) s0 + (1 - alpha^(t+1)) / (1 - alpha).  Pins the inclusive read-out
    (token t's own write counts) and that alpha_0 decays the initial state."""
    one = np.ones((1, 1, L, 1))
    g = np.full((1, 1, L, 1), math.log(alpha))
    o, s = fwd(one, one, one, g=g, gate="keydim", s0=np.full((1, 1, 1, 1), s0))
    t = np.arange(L)
    ref = alpha ** (t + 1) * s0 + (1 - alpha ** (t + 1)) / (1 - alpha)
    return max(rel_err(o.reshape(L), ref), rel_err(s.reshape(1), ref[-1:]))


def pin_chaining(fwd, seed=7, B=2, H=2, L1=17, L2=11, dk=4, dv=5):
    """run(L1 + L2) equals run(L1) followed by run(L2) from its final state (the state
    is the whole history).  Returns the max abs difference (0 in the same op order)."""
    q, k, v, g, S0 = rng_inputs(seed, B, H, L1 + L2, dk, dv, gate="keydim", s0=True)
    o, s = fwd(q, k, v, g=g, gate="keydim", s0=S0)
    oa, sa = fwd(q[:, :, :L1], k[:, :, :L1], v[:, :, :L1], g=g[:, :, :L1], gate="keydim", s0=S0)
    ob, sb = fwd(q[:, :, L1:], k[:, :, L1:], v[:, :, L1:], g=g[:, :, L1:], gate="keydim", s0=sa)
    return float(max(np.max(np.abs(np.concatenate([oa, ob], axis=2) - o)), np.max(np.abs(sb - s))))


def pin_positive_monotone(fwd, seed=8, L=40, dk=4, dv=3):
    """phi = elu+1 is positive; with alpha = 1, v = 1 and the same query at every step,
    each output entry is strictly increasing in t.  Returns the smallest increment
    (must be > 0)."""
    r = np.random.default_rng(seed)
    q = np.repeat(r.standard_normal((1, 1, 1, dk)), L, axis=2)
    k = r.standard_normal((1, 1, L, dk))
    v = np.ones((1, 1, L, dv))
    o, _ = fwd(q, k, v, feature_map="elu1")
    return float(np.min(np.diff(o[0, 0], axis=0)))


# ---- the normalised form ("Transformers are RNNs" notes: numerator over denominator,
# both with the feature map; with gates the denominator state decays like S) ----

def pin_norm_quadratic(fwd_norm, seed=20, fm="elu1", B=2, H=2, L=29, dk=5, dv=4):
    """alpha = 1: o_t = (W V)_t / (W 1)_t with W = (phi(Q) phi(K)^T) (.) L, L_ts = [s <= t]."""
    q, k, v, _, _ = rng_inputs(seed, B, H, L, dk, dv)
    o, _, _ = fwd_norm(q, k, v, feature_map=fm)
    Lm = np.tril(np.ones((L, L)))
    worst = 0.0
    for b in range(B):
        for h in range(H):
            W = (_phi(q[b, h], fm) @ _phi(k[b, h], fm).T) * Lm
            worst = max(worst, rel_err(o[b, h], (W @ v[b, h]) / W.sum(axis=1, keepdims=True)))
    return worst


def pin_norm_unrolled(fwd_norm, seed=21, gate="keydim", B=2, H=2, L=19, dk=4, dv=3):
    """Gated, with initial states: numerator and denominator each in the unrolled form
    (the denominator is the numerator of a value that is 1 in every token, its
    initial state the column z0), and the final z as the explicit sum
    z_L = sum_s phi(k_s) (.) prod_{m>s} alpha_m + prod_m alpha_m (.) z0."""
    q, k, v, g, S0 = rng_inputs(seed, B, H, L, dk, dv, gate=gate, s0=True)
    r = np.random.default_rng(seed + 1000)
    z0 = r.random((B, H, dk)) + 0.5
    qf, kf = _phi(q, "elu1"), _phi(k, "elu1")
    o, _, z = fwd_norm(q, k, v, g=g, gate=gate, feature_map="elu1", s0=S0, z0=z0)
    num = unrolled_reference(qf, kf, v, g, gate, S0)
    den = unrolled_reference(qf, kf, np.ones((B, H, L, 1)), g, gate, z0[..., None])
    worst = rel_err(o, num / den)
    for b in range(B):
        for h in range(H):
            if gate == "keydim":
                alpha = np.exp(g[b, h])
            elif gate == "scalar":
                alpha = np.repeat(np.exp(g[b, h])[:, None], dk, axis=1)
            else:
                alpha = np.ones((L, dk))
            zz = np.prod(alpha, axis=0) * z0[b, h]
            for s_ in range(L):
                zz = zz + kf[b, h, s_] * np.prod(alpha[s_ + 1:], axis=0)
            worst = max(worst, rel_err(z[b, h], zz))
    return worst


def pin_norm_constant_value(fwd_norm, seed=22, B=2, H=2, L=17, dk=3, dv=4):
    """Every value equal to one vector c, zero initial states: every output is c (a
    weighted average of copies of c), with any gate and positive features."""
    q, k, _, g, _ = rng_inputs(seed, B, H, L, dk, dv, gate="keydim")
    c = np.array([0.5, -2.0, 3.25, 1.0])[:dv]
    v = np.broadcast_to(c, (B, H, L, dv)).copy()
    o, _, _ = fwd_norm(q, k, v, g=g, gate="keydim", feature_map="elu1")
    return rel_err(o, np.broadcast_to(c, o.shape))


def pin_norm_chaining(fwd_norm, seed=23, B=2, H=2, L1=13, L2=9, dk=4, dv=3):
    """run(L1 + L2) equals run(L1) followed by run(L2) from its (S, z): the same
    operations in the same order, so bit for bit."""
    q, k, v, g, S0 = rng_inputs(seed, B, H, L1 + L2, dk, dv, gate="scalar", s0=True)
    o, s, z = fwd_norm(q, k, v, g=g, gate="scalar", feature_map="elu1", s0=S0)
    o1, s1, z1 = fwd_norm(q[:, :, :L1], k[:, :, :L1], v[:, :, :L1], g=g[:, :, :L1], gate="scalar",
                          feature_map="elu1", s0=S0)
    o2, s2, z2 = fwd_norm(q[:, :, L1:], k[:, :, L1:], v[:, :, L1:], g=g[:, :, L1:], gate="scalar",
                          feature_map="elu1", s0=s1, z0=z1)
    with np.errstate(invalid="ignore"):            # a broken oracle may give NaN: reported as NaN
        return float(max(np.abs(o - np.concatenate([o1, o2], axis=2)).max(), np.abs(s - s2).max(),
                         np.abs(z - z2).max()))


def norm_convexity_violation(fwd_norm, seed=24, B=2, H=2, L=31, dk=4, dv=5):
    """Positive features and gates in (0, 1]: each output coordinate is a convex
    combination of that coordinate over the values so far.  Returns the largest
    amount by which an output leaves [min_{s<=t} v_s, max_{s<=t} v_s] (0 when none)."""
    q, k, v, g, _ = rng_inputs(seed, B, H, L, dk, dv, gate="keydim")
    o, _, _ = fwd_norm(q, k, v, g=g, gate="keydim", feature_map="elu1")
    lo = np.minimum.accumulate(v, axis=2)
    hi = np.maximum.accumulate(v, axis=2)
    return float(max(0.0, (lo - o).max(), (o - hi).max()))


NORM_ERROR_PINS = {
    # name: (callable on forward_norm, tolerance)
    "norm_quadratic_elu1": (pin_norm_quadratic, 1e-12),
    "norm_unrolled_keydim": (pin_norm_unrolled, 1e-12),
    "norm_unrolled_scalar": (lambda f: pin_norm_unrolled(f, seed=25, gate="scalar"), 1e-12),
    "norm_unrolled_none": (lambda f: pin_norm_unrolled(f, seed=26, gate=None), 1e-12),
    "norm_constant_value": (pin_norm_constant_value, 1e-14),
    "norm_chaining": (pin_norm_chaining, 0.0),
    "norm_convexity": (norm_convexity_violation, 1e-12),
}


ALL_ERROR_PINS = {
    # name: (callable, tolerance); each returns an error that must stay below tolerance
    "feature_map_points": (pin_feature_map_points, 1e-15),
    "quadratic_masked": (pin_quadratic_masked, 1e-12),
    "quadratic_masked_elu1": (lambda f: pin_quadratic_masked(f, seed=10, fm="elu1"), 1e-12),
    "cumsum_last_token": (pin_cumsum_and_last_token, 1e-12),
    "cumsum_last_token_elu1": (lambda f: pin_cumsum_and_last_token(f, seed=11, fm="elu1"), 1e-12),
    "unrolled_keydim": (pin_unrolled, 1e-12),
    "unrolled_scalar": (lambda f: pin_unrolled(f, seed=12, gate="scalar"), 1e-12),
    "exact_rational": (pin_exact_rational, 1e-14),
    "scalar_broadcast": (pin_scalar_is_broadcast_keydim, 1e-15),
    "retnet_geometric": (pin_retnet_geometric, 1e-12),
    "vanishing_gate": (pin_vanishing_gate, 1e-15),
    "geometric_closed_form": (pin_geometric_closed_form, 1e-14),
    "chaining": (pin_chaining, 0.0),
}


# ---- the delta rule ("Attention is recurrent", Delta attention and its Prefill):
# the write is the prediction error scaled by beta; prefill is one triangular system ----

def delta_inputs(seed, B, H, L, dk, dv, s0=False):
    """Unit-norm keys and queries (the usual normalisation for the delta rule, which
    keeps every I - beta k k^T a contraction for beta in [0, 1]) and beta in (0, 1)."""
    r = np.random.default_rng(seed)
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q = unit(r.standard_normal((B, H, L, dk)))
    k = unit(r.standard_normal((B, H, L, dk)))
    v = r.standard_normal((B, H, L, dv))
    beta = r.uniform(0.05, 0.95, size=(B, H, L))
    S0 = r.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, beta, S0


def pin_delta_triangular(fwd_delta, seed=30, with_s0=True, B=2, H=2, L=23, dk=5, dv=4):
    """The whole prompt as one lower-triangular system: with T = I + tril(diag(beta) K K^T, -1),
    the writes are U = T^{-1} diag(beta) (V - K S0), the outputs O = Q S0 + tril(Q K^T) U
    (the read-out includes the token's own write) and the final state S0 + K^T U.
    Solved with numpy's dense solver, not by substitution."""
    q, k, v, beta, S0 = delta_inputs(seed, B, H, L, dk, dv, s0=with_s0)
    o, s = fwd_delta(q, k, v, beta, s0=S0)
    worst = 0.0
    for b in range(B):
        for h in range(H):
            K, Q, V, be = k[b, h], q[b, h], v[b, h], beta[b, h]
            s0 = S0[b, h] if S0 is not None else np.zeros((dk, dv))
            T = np.eye(L) + np.tril(be[:, None] * (K @ K.T), -1)
            U = np.linalg.solve(T, be[:, None] * (V - K @ s0))
            worst = max(worst, rel_err(o[b, h], Q @ s0 + np.tril(Q @ K.T) @ U),
                        rel_err(s[b, h], s0 + K.T @ U))
    return worst


def pin_delta_zero_strength(fwd_delta, seed=31, B=2, H=2, L=11, dk=4, dv=3):
    """beta = 0 writes nothing: S stays S0 and o_t = S0^T q_t."""
    q, k, v, _, S0 = delta_inputs(seed, B, H, L, dk, dv, s0=True)
    o, s = fwd_delta(q, k, v, np.zeros((B, H, L)), s0=S0)
    return max(float(np.abs(s - S0).max()),
               rel_err(o, np.einsum("bhli,bhij->bhlj", q, S0)))


def pin_delta_overwrite(fwd_delta, seed=32, B=1, H=2, L=20, dk=6, dv=3):
    """beta = 1 with keys drawn from an orthonormal basis: each write replaces the
    value stored under its key exactly.  Reading with q_t = k_t returns v_t; at the
    end S^T e = the last value written to basis key e, and S is unchanged along
    basis keys never written."""
    r = np.random.default_rng(seed)
    basis, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    idx = r.integers(0, dk - 1, size=(B, H, L))          # the last basis key is never written
    k = basis.T[idx]                                      # rows are basis vectors
    v = r.standard_normal((B, H, L, dv))
    S0 = r.standard_normal((B, H, dk, dv))
    o, s = fwd_delta(k.copy(), k, v, np.ones((B, H, L)), s0=S0)
    worst = rel_err(o, v)
    for b in range(B):
        for h in range(H):
            for e in range(dk):
                hits = np.nonzero(idx[b, h] == e)[0]
                want = v[b, h, hits[-1]] if hits.size else S0[b, h].T @ basis[:, e]
                worst = max(worst, float(np.abs(s[b, h].T @ basis[:, e] - want).max()))
    return worst


def pin_delta_moving_average(fwd_delta, seed=33, L=30, dv=3):
    """d_k = 1, every key and query 1: the delta rule is the exponential moving average
    s_n = (1 - beta_n) s_{n-1} + beta_n v_n, here in its explicit product form
    s_n = prod_{m<=n} (1 - beta_m) s0 + sum_{i<=n} beta_i v_i prod_{i<m<=n} (1 - beta_m)."""
    r = np.random.default_rng(seed)
    beta = r.uniform(0.0, 1.0, size=(1, 1, L))
    v = r.standard_normal((1, 1, L, dv))
    S0 = r.standard_normal((1, 1, 1, dv))
    ones = np.ones((1, 1, L, 1))
    o, s = fwd_delta(ones, ones, v, beta, s0=S0)
    keep = 1.0 - beta[0, 0]
    want = np.zeros((L, dv))
    for n in range(L):
        acc = np.prod(keep[:n + 1]) * S0[0, 0, 0]
        for i in range(n + 1):
            acc = acc + beta[0, 0, i] * v[0, 0, i] * np.prod(keep[i + 1:n + 1])
        want[n] = acc
    return max(rel_err(o[0, 0], want), rel_err(s[0, 0, 0], want[-1]))


def pin_delta_chaining(fwd_delta, seed=34, B=2, H=2, L1=12, L2=9, dk=4, dv=3):
    """run(L1 + L2) equals run(L1) followed by run(L2) from its final state, bit for bit."""
    q, k, v, beta, S0 = delta_inputs(seed, B, H, L1 + L2, dk, dv, s0=True)
    o, s = fwd_delta(q, k, v, beta, s0=S0)
    o1, s1 = fwd_delta(q[:, :, :L1], k[:, :, :L1], v[:, :, :L1], beta[:, :, :L1], s0=S0)
    o2, s2 = fwd_delta(q[:, :, L1:], k[:, :, L1:], v[:, :, L1:], beta[:, :, L1:], s0=s1)
    with np.errstate(invalid="ignore"):
        return float(max(np.abs(o - np.concatenate([o1, o2], axis=2)).max(), np.abs(s - s2).max()))


DELTA_ERROR_PINS = {
    # name: (callable on forward_delta, tolerance)
    "delta_triangular": (pin_delta_triangular, 1e-12),
    "delta_triangular_zero_init": (lambda f: pin_delta_triangular(f, seed=35, with_s0=False), 1e-12),
    "delta_zero_strength": (pin_delta_zero_strength, 1e-15),
    "delta_overwrite": (pin_delta_overwrite, 1e-13),
    "delta_moving_average": (pin_delta_moving_average, 1e-13),
    "delta_chaining": (pin_delta_chaining, 0.0),
}


# ---- the input-side gate producer ("Gated Linear Attention", Recurrent Form:
# alpha_t = sigmoid(W_up W_down x_t); log-gates in the prefill layout) ----

def _gate_inputs(seed, B, L, dm, r, H, dk, scale=1.0):
    rr = np.random.default_rng(seed)
    x = rr.standard_normal((B, L, dm))
    wd = rr.standard_normal((r, dm)) * scale / math.sqrt(dm)
    wu = rr.standard_normal((H * dk, r)) * scale / math.sqrt(r)
    return x, wd, wu


def pin_gate_brute_force(gate, seed=40, B=2, L=3, dm=5, r=2, H=2, dk=3, tau=1.0):
    """Explicit sums over d_model and r in Python floats, and the textbook
    log(1 / (1 + e^-z)) (the values here stay well inside its safe range)."""
    x, wd, wu = _gate_inputs(seed, B, L, dm, r, H, dk)
    g = gate(x, wd, wu, H, dk, tau)
    worst = 0.0
    for b in range(B):
        for t in range(L):
            zd = [sum(wd[j][m] * x[b][t][m] for m in range(dm)) for j in range(r)]
            for h in range(H):
                for i in range(dk):
                    z = sum(wu[h * dk + i][j] * zd[j] for j in range(r))
                    want = math.log(1.0 / (1.0 + math.exp(-z))) / tau
                    worst = max(worst, abs(g[b, h, t, i] - want) / max(abs(want), 1e-300))
    return worst


def pin_gate_zero_input(gate, seed=41, B=1, L=4, dm=8, r=4, H=2, dk=4, tau=16.0):
    """x = 0 (or zero weights) gives z = 0: every gate is sigmoid(0) = 1/2, g = -ln 2 / tau."""
    _, wd, wu = _gate_inputs(seed, B, L, dm, r, H, dk)
    g1 = gate(np.zeros((B, L, dm)), wd, wu, H, dk, tau)
    g2 = gate(np.ones((B, L, dm)), np.zeros_like(wd), wu, H, dk, tau)
    want = -math.log(2.0) / tau
    return float(max(np.abs(g1 - want).max(), np.abs(g2 - want).max()) / abs(want))


def pin_gate_rank_one_select(gate, seed=42, B=2, L=5, dm=6, r=3, H=2, dk=4):
    """W_down picks input coordinate c into rank slot 0, W_up copies slot 0 to output
    n scaled by s_n: z_t[n] = s_n x_t[c], so g[b, h, t, i] = log sigmoid(s_{h d_k+i} x[b, t, c])."""
    rr = np.random.default_rng(seed)
    x = rr.standard_normal((B, L, dm)) * 3.0
    c = 2
    wd = np.zeros((r, dm))
    wd[0, c] = 1.0
    s = rr.standard_normal(H * dk)
    wu = np.zeros((H * dk, r))
    wu[:, 0] = s
    g = gate(x, wd, wu, H, dk, 1.0)
    z = x[:, :, c][:, None, :, None] * s.reshape(H, dk)[None, :, None, :]
    want = np.log(1.0 / (1.0 + np.exp(-z)))
    return rel_err(g, want)


def pin_gate_extremes(gate):
    """Large |z|: log sigmoid(z) -> z for z -> -inf and -> -e^-z for z -> +inf; each
    checked to relative accuracy (a naive log(sigmoid) would give -inf / 0)."""
    zs = np.array([-800.0, -60.0, -30.0, 30.0, 60.0, 700.0])
    x = zs.reshape(1, len(zs), 1)
    g = gate(x, np.ones((1, 1)), np.ones((1, 1)), 1, 1, 1.0)[0, 0, :, 0]
    neg, pos = np.minimum(zs, 0.0), np.maximum(zs, 0.0)
    want = np.where(zs < 0, neg - np.exp(neg), -np.exp(-pos) + np.exp(-2 * pos) / 2)   # series
    return float(np.max(np.abs(g - want) / np.abs(want)))


def pin_gate_sigmoid_identity(gate, seed=43, B=2, L=7, dm=16, r=4, H=3, dk=4, tau=4.0):
    """exp(tau g) is the logistic function of z, here via scipy.special.expit, and lies
    in (0, 1)."""
    from scipy.special import expit
    x, wd, wu = _gate_inputs(seed, B, L, dm, r, H, dk, scale=2.0)
    g = gate(x, wd, wu, H, dk, tau)
    z = (x @ wd.T @ wu.T).reshape(B, L, H, dk).transpose(0, 2, 1, 3)
    a = np.exp(tau * g)
    return max(rel_err(a, expit(z)), float(max(0.0, a.max() - 1.0, -a.min())))


GATE_ERROR_PINS = {
    # name: (callable on the gate producer, tolerance)
    "gate_brute_force": (pin_gate_brute_force, 1e-12),
    "gate_brute_force_tau": (lambda f: pin_gate_brute_force(f, seed=44, tau=16.0), 1e-12),
    "gate_zero_input": (pin_gate_zero_input, 1e-14),
    "gate_rank_one_select": (pin_gate_rank_one_select, 1e-12),
    "gate_extremes": (pin_gate_extremes, 1e-14),
    "gate_sigmoid_identity": (pin_gate_sigmoid_identity, 1e-13),
}


# ---- the outer-product gate ("Gated Linear Attention", Recurrent Form: the low-rank
# parameterisation G_t = alpha_t beta_t^T of the gate G_t (.) S_{t-1}) ----

def _outer_inputs(seed, B, H, L, dk, dv, s0=True, scale=0.3):
    q, k, v, g, S0 = rng_inputs(seed, B, H, L, dk, dv, gate="keydim", s0=s0, g_scale=scale)
    gv = -scale * np.random.default_rng(seed + 500).random((B, H, L, dv))
    return q, k, v, g, gv, S0


def pin_outer_unrolled(fwd_outer, seed=50, fm=None, B=2, H=2, L=17, dk=4, dv=3):
    """Explicit products: a write at token i reaches token n scaled by
    prod_{m=i+1..n} alpha_m[c] beta_m[j] in entry (c, j); the initial state by the
    product over all m <= n.  Outputs and the final state are both checked."""
    q, k, v, g, gv, S0 = _outer_inputs(seed, B, H, L, dk, dv)
    o, s = fwd_outer(q, k, v, g, gv, feature_map=fm, s0=S0)
    qf, kf = _phi(q, fm), _phi(k, fm)
    al, be = np.exp(g), np.exp(gv)
    worst = 0.0
    for b in range(B):
        for h in range(H):
            for n in range(L):
                Sn = S0[b, h] * np.outer(np.prod(al[b, h, :n + 1], axis=0), np.prod(be[b, h, :n + 1], axis=0))
                for i in range(n + 1):
                    w = np.outer(np.prod(al[b, h, i + 1:n + 1], axis=0), np.prod(be[b, h, i + 1:n + 1], axis=0))
                    Sn = Sn + np.outer(kf[b, h, i], v[b, h, i]) * w
                worst = max(worst, rel_err(o[b, h, n], qf[b, h, n] @ Sn))
                if n == L - 1:
                    worst = max(worst, rel_err(s[b, h], Sn))
    return worst


def pin_outer_uniform_is_scalar_mask(fwd_outer, seed=51, B=2, H=2, L=23, dk=5, dv=4):
    """alpha_t = a_t 1 and beta_t = b_t 1 make G_t = (a_t b_t) 1 1^T, the Mamba2 scalar
    gate: O = ((Q K^T) (.) D) V with the decay mask D_ts = prod_{m=s+1..t} a_m b_m for
    s <= t (0 above the diagonal), evaluated as a matrix."""
    q, k, v, _, _, _ = _outer_inputs(seed, B, H, L, dk, dv, s0=False)
    r = np.random.default_rng(seed + 1)
    la = -0.3 * r.random((B, H, L))
    lb = -0.2 * r.random((B, H, L))
    g = np.repeat(la[..., None], dk, axis=3)
    gv = np.repeat(lb[..., None], dv, axis=3)
    o, _ = fwd_outer(q, k, v, g, gv)
    worst = 0.0
    for b in range(B):
        for h in range(H):
            c = np.cumsum(la[b, h] + lb[b, h])
            D = np.tril(np.exp(c[:, None] - c[None, :]))
            worst = max(worst, rel_err(o[b, h], ((q[b, h] @ k[b, h].T) * D) @ v[b, h]))
    return worst


def pin_outer_value_gate_only(fwd_outer, seed=52, L=9, dv=3):
    """d_k = 1, q = k = 1, alpha = 1: each value column j is an independent geometric
    accumulator, s_n[j] = beta_n[j] s_{n-1}[j] + v_n[j], evaluated in closed form as a
    sum of products."""
    r = np.random.default_rng(seed)
    v = r.standard_normal((1, 1, L, dv))
    gv = -0.5 * r.random((1, 1, L, dv))
    S0 = r.standard_normal((1, 1, 1, dv))
    ones = np.ones((1, 1, L, 1))
    o, s = fwd_outer(ones, ones, v, np.zeros((1, 1, L, 1)), gv, s0=S0)
    be = np.exp(gv[0, 0])
    want = np.zeros((L, dv))
    for n in range(L):
        acc = S0[0, 0, 0] * np.prod(be[:n + 1], axis=0)
        for i in range(n + 1):
            acc = acc + v[0, 0, i] * np.prod(be[i + 1:n + 1], axis=0)
        want[n] = acc
    return max(rel_err(o[0, 0], want), rel_err(s[0, 0, 0], want[-1]))


def pin_outer_chaining(fwd_outer, seed=53, B=2, H=2, L1=11, L2=8, dk=4, dv=5):
    """run(L1 + L2) equals run(L1) followed by run(L2) from its final state, bit for bit."""
    q, k, v, g, gv, S0 = _outer_inputs(seed, B, H, L1 + L2, dk, dv)
    o, s = fwd_outer(q, k, v, g, gv, feature_map="elu1", s0=S0)
    a, b_ = slice(0, L1), slice(L1, L1 + L2)
    o1, s1 = fwd_outer(q[:, :, a], k[:, :, a], v[:, :, a], g[:, :, a], gv[:, :, a], feature_map="elu1", s0=S0)
    o2, s2 = fwd_outer(q[:, :, b_], k[:, :, b_], v[:, :, b_], g[:, :, b_], gv[:, :, b_], feature_map="elu1", s0=s1)
    with np.errstate(invalid="ignore"):
        return float(max(np.abs(o - np.concatenate([o1, o2], axis=2)).max(), np.abs(s - s2).max()))


OUTER_ERROR_PINS = {
    # name: (callable on forward_outer, tolerance)
    "outer_unrolled": (pin_outer_unrolled, 1e-12),
    "outer_unrolled_elu1": (lambda f: pin_outer_unrolled(f, seed=54, fm="elu1"), 1e-12),
    "outer_uniform_is_scalar_mask": (pin_outer_uniform_is_scalar_mask, 1e-12),
    "outer_value_gate_only": (pin_outer_value_gate_only, 1e-13),
    "outer_chaining": (pin_outer_chaining, 0.0),
}
