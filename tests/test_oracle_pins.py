"""CPU tests: the fp64 oracle against the independent forms in ``pins.py`` and the
stored worked example under ``golden/``."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prefill_4token.json")


@pytest.mark.parametrize("name", sorted(pins.ALL_ERROR_PINS))
def test_oracle_pin(name):
    fn, tol = pins.ALL_ERROR_PINS[name]
    err = fn(oracle.forward)
    assert err <= tol, "%s: error %.3e above %.1e" % (name, err, tol)


@pytest.mark.parametrize("name", sorted(pins.NORM_ERROR_PINS))
def test_oracle_norm_pin(name):
    fn, tol = pins.NORM_ERROR_PINS[name]
    err = fn(oracle.forward_norm)
    assert err <= tol, "%s: error %.3e above %.1e" % (name, err, tol)


@pytest.mark.parametrize("name", sorted(pins.DELTA_ERROR_PINS))
def test_oracle_delta_pin(name):
    fn, tol = pins.DELTA_ERROR_PINS[name]
    err = fn(oracle.forward_delta)
    assert err <= tol, "%s: error %.3e above %.1e" % (name, err, tol)


def test_oracle_delta_empty_and_bad_strength():
    q, k, v, beta, S0 = pins.delta_inputs(36, 2, 2, 0, 4, 3, s0=True)
    o, s = oracle.forward_delta(q, k, v, beta, s0=S0)
    assert o.shape == (2, 2, 0, 3) and np.array_equal(s, S0)
    q, k, v, beta, _ = pins.delta_inputs(37, 1, 2, 5, 4, 3)
    with pytest.raises(ValueError):
        oracle.forward_delta(q, k, v, beta[..., :4])
    with pytest.raises(ValueError):
        oracle.forward_delta(q, k, v, None)


def test_oracle_delta_threads_agree_bitwise():
    q, k, v, beta, S0 = pins.delta_inputs(38, 3, 5, 17, 6, 7, s0=True)
    o1, s1 = oracle.forward_delta(q, k, v, beta, s0=S0, nthreads=1)
    o8, s8 = oracle.forward_delta(q, k, v, beta, s0=S0, nthreads=8)
    assert np.array_equal(o1, o8) and np.array_equal(s1, s8)


@pytest.mark.parametrize("name", sorted(pins.OUTER_ERROR_PINS))
def test_oracle_outer_pin(name):
    fn, tol = pins.OUTER_ERROR_PINS[name]
    err = fn(oracle.forward_outer)
    assert err <= tol, "%s: error %.3e above %.1e" % (name, err, tol)


def test_oracle_outer_with_unit_value_gate_is_keydim():
    """beta = 1 (gv = 0) leaves the key-dim gated recurrence, bit for bit."""
    q, k, v, g, S0 = pins.rng_inputs(28, 2, 2, 15, 4, 5, gate="keydim", s0=True)
    o1, s1 = oracle.forward(q, k, v, g=g, gate="keydim", s0=S0)
    o2, s2 = oracle.forward_outer(q, k, v, g, np.zeros((2, 2, 15, 5)), s0=S0)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_oracle_norm_matches_unnormalised_state():
    """The normalised entry carries S exactly as the plain one does."""
    q, k, v, g, S0 = pins.rng_inputs(27, 2, 3, 21, 5, 4, gate="keydim", s0=True)
    _, s1 = oracle.forward(q, k, v, g=g, gate="keydim", feature_map="elu1", s0=S0)
    _, s2, _ = oracle.forward_norm(q, k, v, g=g, gate="keydim", feature_map="elu1", s0=S0)
    assert np.array_equal(s1, s2)


def test_oracle_positive_monotone():
    assert pins.pin_positive_monotone(oracle.forward) > 0.0


def test_oracle_threads_agree_bitwise():
    q, k, v, g, S0 = pins.rng_inputs(21, 3, 5, 19, 6, 7, gate="keydim", s0=True)
    o1, s1 = oracle.forward(q, k, v, g=g, gate="keydim", s0=S0, nthreads=1)
    o8, s8 = oracle.forward(q, k, v, g=g, gate="keydim", s0=S0, nthreads=8)
    assert np.array_equal(o1, o8) and np.array_equal(s1, s8)


def test_oracle_empty_sequence_returns_initial_state():
    q, k, v, g, S0 = pins.rng_inputs(22, 2, 2, 0, 4, 3, gate="keydim", s0=True)
    o, s = oracle.forward(q, k, v, g=g, gate="keydim", s0=S0)
    assert o.shape == (2, 2, 0, 3) and np.array_equal(s, S0)


def test_oracle_rejects_bad_shapes():
    q, k, v, g, _ = pins.rng_inputs(23, 1, 1, 4, 3, 2, gate="keydim")
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, g=g[..., 0], gate="keydim")
    with pytest.raises(ValueError):
        oracle.forward(q, k[..., :2], v)


def _exact_unrolled(case):
    """Exact rational outputs of the stored example via the unrolled form."""
    q, k, v = (np.array(case[x], dtype=object) for x in ("q", "k", "v"))
    a = [[Fraction(x) for x in row] for row in case["alpha"]]
    L, dk = q.shape
    dv = v.shape[1]
    out = []
    for n in range(L):
        row = []
        for j in range(dv):
            tot = Fraction(0)
            for i in range(n + 1):
                for c in range(dk):
                    w = Fraction(1)
                    for m in range(i + 1, n + 1):
                        w *= a[m][c]
                    tot += Fraction(q[n, c]) * Fraction(k[i, c]) * w * Fraction(v[i, j])
            row.append(tot)
        out.append(row)
    return np.array([[float(x) for x in r] for r in out])


def test_golden_prefill_4token():
    """A four-token prompt x_0..x_3 prefilled in one pass (the shape of the worked
    example in "Attention is recurrent", Prefill, whose numbers did not survive):
    the stored outputs were written by ``golden/make_golden.py`` from the oracle; they
    must match exact rational arithmetic and the oracle must still reproduce them."""
    with open(GOLDEN) as f:
        case = json.load(f)
    want = np.array(case["o"], dtype=np.float64)
    exact = _exact_unrolled(case)
    assert pins.rel_err(want, exact) < 1e-14
    L, dk = len(case["q"]), len(case["q"][0])
    dv = len(case["v"][0])
    alpha = np.array([[float(Fraction(x)) for x in r] for r in case["alpha"]])
    o, _ = oracle.forward(np.array(case["q"], float).reshape(1, 1, L, dk),
                          np.array(case["k"], float).reshape(1, 1, L, dk),
                          np.array(case["v"], float).reshape(1, 1, L, dv),
                          g=np.log(alpha).reshape(1, 1, L, dk), gate="keydim")
    assert pins.rel_err(o[0, 0], want) < 1e-14


def _gauss_jordan(A, B):
    """Exact solution X of A X = B in Fractions by Gauss-Jordan elimination with row
    pivoting (a general solver: it does not use A's triangular structure)."""
    n, m = len(A), len(B[0])
    M = [list(A[i]) + list(B[i]) for i in range(n)]
    for c in range(n):
        piv = next(r for r in range(c, n) if M[r][c] != 0)
        M[c], M[piv] = M[piv], M[c]
        inv = 1 / M[c][c]
        M[c] = [x * inv for x in M[c]]
        for r in range(n):
            if r != c and M[r][c] != 0:
                f = M[r][c]
                M[r] = [x - f * y for x, y in zip(M[r], M[c])]
    return [row[n:] for row in M]


def test_golden_delta_4token():
    """A four-token delta prefill (the shape of the page's Delta attention / Prefill
    example, whose numbers did not survive): the stored outputs, written by
    ``golden/make_golden.py`` from the oracle, must equal exact rational arithmetic on
    the page's lower-triangular system (T U = diag(beta) V with
    T = I + tril(diag(beta) K K^T, -1), O = tril(Q K^T) U, S = K^T U), solved by a
    general elimination; and the oracle must still reproduce them."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "delta_4token.json")) as f:
        case = json.load(f)
    Q = [[Fraction(x) for x in r] for r in case["q"]]
    K = [[Fraction(x) for x in r] for r in case["k"]]
    V = [[Fraction(x) for x in r] for r in case["v"]]
    be = [Fraction(x) for x in case["beta"]]
    L, dk, dv = len(Q), len(Q[0]), len(V[0])
    dot = lambda a, b: sum(x * y for x, y in zip(a, b))
    T = [[Fraction(int(i == j)) + (be[i] * dot(K[i], K[j]) if j < i else 0) for j in range(L)] for i in range(L)]
    U = _gauss_jordan(T, [[be[i] * V[i][j] for j in range(dv)] for i in range(L)])
    O = [[sum(dot(Q[t], K[s]) * U[s][j] for s in range(t + 1)) for j in range(dv)] for t in range(L)]
    S = [[sum(K[s][i] * U[s][j] for s in range(L)) for j in range(dv)] for i in range(dk)]
    exact_o = np.array([[float(x) for x in r] for r in O])
    exact_s = np.array([[float(x) for x in r] for r in S])
    want_o, want_s = np.array(case["o"]), np.array(case["s_final"])
    assert pins.rel_err(want_o, exact_o) < 1e-14 and pins.rel_err(want_s, exact_s) < 1e-14
    o, s = oracle.forward_delta(np.array(case["q"], float).reshape(1, 1, L, dk),
                                np.array(case["k"], float).reshape(1, 1, L, dk),
                                np.array(case["v"], float).reshape(1, 1, L, dv),
                                np.array([float(x) for x in be]).reshape(1, 1, L))
    assert pins.rel_err(o[0, 0], want_o) < 1e-14 and pins.rel_err(s[0, 0], want_s) < 1e-14
