"""Python binding of the fp64 CPU oracle (``gla_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The product path never
does, and this module imports nothing from the product package.

The oracle is the token-by-token recurrence of the pages ("Attention is
recurrent", sections "Linear attention" and "Gated linear attention"; "Gated
Linear Attention", section "GLA / Recurrent Form"), run in double precision:

    S_t = Diag(alpha_t) S_{t-1} + phi(k_t) v_t^T,   o_t = S_t^T phi(q_t)

with alpha_t = exp(g_t) per key dimension, a scalar exp(g_t) for every key
dimension, or 1.  Inputs are upcast exactly to float64 from whatever bits the
caller holds (bf16 and fp32 both convert exactly).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

GATE_MODES = {None: 0, "none": 0, "keydim": 1, "scalar": 2}
FEATURE_MAPS = {None: 0, "identity": 0, "elu1": 1}

_libs = {}


def compile_source(src: str, out: str) -> str:
    """Compile one C source of the oracle into a shared library with gcc (no fast-math)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
                           "-o", tmp, src, "-lm", "-lpthread"])
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile ``gla_oracle.c`` into ``liboracle.so`` (always when ``force``)."""
    if force or not os.path.exists(_LIB_PATH):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


def _load(lib_path=None):
    if lib_path is None:
        build()
        lib_path = _LIB_PATH
    if lib_path not in _libs:
        lib = ctypes.CDLL(lib_path)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.gla_oracle_forward.argtypes = [dp, dp, dp, dp, ctypes.c_int, ctypes.c_int, dp, dp, dp,
                                           ctypes.c_long, ctypes.c_long, ctypes.c_long,
                                           ctypes.c_long, ctypes.c_long, ctypes.c_int]
        lib.gla_oracle_forward.restype = ctypes.c_int
        lib.gla_oracle_forward_norm.argtypes = [dp, dp, dp, dp, ctypes.c_int, ctypes.c_int, dp, dp, dp,
                                                dp, dp, ctypes.c_long, ctypes.c_long, ctypes.c_long,
                                                ctypes.c_long, ctypes.c_long, ctypes.c_int]
        lib.gla_oracle_forward_norm.restype = ctypes.c_int
        lib.gla_oracle_delta.argtypes = [dp, dp, dp, dp, dp, dp, dp, ctypes.c_long, ctypes.c_long,
                                         ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_int]
        lib.gla_oracle_delta.restype = ctypes.c_int
        lib.gla_oracle_forward_outer.argtypes = [dp, dp, dp, dp, dp, ctypes.c_int, dp, dp, dp, ctypes.c_long,
                                                 ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long,
                                                 ctypes.c_int]
        lib.gla_oracle_forward_outer.restype = ctypes.c_int
        _libs[lib_path] = lib
    return _libs[lib_path]


def _f64(x):
    """Exact upcast to a C-contiguous float64 numpy array (accepts torch tensors)."""
    if x is None:
        return None
    if hasattr(x, "detach"):                       # torch tensor, any device / dtype
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:                          # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _prepare(q, k, v, g, gate, s0):
    q, k, v, g, s0 = _f64(q), _f64(k), _f64(v), _f64(g), _f64(s0)
    if q.ndim != 4 or k.shape != q.shape or v.ndim != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("oracle: q, k must be [B,H,L,d_k] and v [B,H,L,d_v]")
    B, H, L, dk = q.shape
    dv = v.shape[3]
    mode = GATE_MODES[gate]
    if mode == 1 and (g is None or g.shape != (B, H, L, dk)):
        raise ValueError("oracle: key-dim gate needs g of shape [B,H,L,d_k]")
    if mode == 2 and (g is None or g.shape != (B, H, L)):
        raise ValueError("oracle: scalar gate needs g of shape [B,H,L]")
    if mode == 0:
        g = None
    if s0 is not None and s0.shape != (B, H, dk, dv):
        raise ValueError("oracle: s0 must be [B,H,d_k,d_v]")
    return q, k, v, g, s0, mode, (B, H, L, dk, dv)


def forward(q, k, v, g=None, gate=None, feature_map=None, s0=None, nthreads=None, lib_path=None):
    """Run the recurrence over every (b, h).

    q, k: [B, H, L, d_k]; v: [B, H, L, d_v]; g: [B, H, L, d_k] for gate="keydim",
    [B, H, L] for gate="scalar", None for no gate; s0: [B, H, d_k, d_v] or None.
    Returns (o [B, H, L, d_v], s_final [B, H, d_k, d_v]) as float64 arrays.
    ``lib_path`` selects another build of the oracle source (the pin tests use it to
    check that planted mistakes are caught); by default the committed source is used.
    """
    q, k, v, g, s0, mode, (B, H, L, dk, dv) = _prepare(q, k, v, g, gate, s0)
    o = np.zeros((B, H, L, dv), dtype=np.float64)
    s = np.zeros((B, H, dk, dv), dtype=np.float64)
    nthreads = default_threads() if nthreads is None else int(nthreads)
    rc = _load(lib_path).gla_oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), mode,
                                    FEATURE_MAPS[feature_map], _ptr(s0), _ptr(o), _ptr(s),
                                    B, H, L, dk, dv, nthreads)
    if rc != 0:
        raise RuntimeError("gla_oracle_forward failed with code %d" % rc)
    return o, s


def forward_norm(q, k, v, g=None, gate=None, feature_map=None, s0=None, z0=None, nthreads=None,
                 lib_path=None):
    """The normalised form ("Transformers are RNNs" notes: weighted sum of values over
    the sum of the weights): as ``forward``, with the normaliser state z carried
    beside S (z_t = alpha_t * z_{t-1} + phi(k_t), o_t = S_t^T phi(q_t) / phi(q_t).z_t).
    z0: [B, H, d_k] or None.  Returns (o, s_final, z_final) as float64 arrays."""
    q, k, v, g, s0, mode, (B, H, L, dk, dv) = _prepare(q, k, v, g, gate, s0)
    z0 = _f64(z0)
    if z0 is not None and z0.shape != (B, H, dk):
        raise ValueError("oracle: z0 must be [B,H,d_k]")
    o = np.zeros((B, H, L, dv), dtype=np.float64)
    s = np.zeros((B, H, dk, dv), dtype=np.float64)
    z = np.zeros((B, H, dk), dtype=np.float64)
    nthreads = default_threads() if nthreads is None else int(nthreads)
    rc = _load(lib_path).gla_oracle_forward_norm(_ptr(q), _ptr(k), _ptr(v), _ptr(g), mode,
                                         FEATURE_MAPS[feature_map], _ptr(s0), _ptr(z0), _ptr(o),
                                         _ptr(s), _ptr(z), B, H, L, dk, dv, nthreads)
    if rc != 0:
        raise RuntimeError("gla_oracle_forward_norm failed with code %d" % rc)
    return o, s, z


def forward_delta(q, k, v, beta, s0=None, nthreads=None, lib_path=None):
    """The delta rule ("Attention is recurrent", Delta attention): u_t = beta_t (v_t -
    S_{t-1}^T k_t), S_t = S_{t-1} + k_t u_t^T, o_t = S_t^T q_t.  beta: [B, H, L];
    s0: [B, H, d_k, d_v] or None.  Returns (o, s_final) as float64 arrays."""
    q, k, v, _, s0, _, (B, H, L, dk, dv) = _prepare(q, k, v, None, None, s0)
    beta = _f64(beta)
    if beta is None or beta.shape != (B, H, L):
        raise ValueError("oracle: beta must be [B,H,L]")
    o = np.zeros((B, H, L, dv), dtype=np.float64)
    s = np.zeros((B, H, dk, dv), dtype=np.float64)
    nthreads = default_threads() if nthreads is None else int(nthreads)
    rc = _load(lib_path).gla_oracle_delta(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(s0), _ptr(o), _ptr(s),
                                          B, H, L, dk, dv, nthreads)
    if rc != 0:
        raise RuntimeError("gla_oracle_delta failed with code %d" % rc)
    return o, s


def forward_outer(q, k, v, g, gv, feature_map=None, s0=None, nthreads=None, lib_path=None):
    """The outer-product gate ("Gated Linear Attention", Recurrent Form, G_t = alpha_t
    beta_t^T): S_t = (alpha_t beta_t^T) (.) S_{t-1} + phi(k_t) v_t^T, o_t = S_t^T phi(q_t),
    with natural-log gates g [B, H, L, d_k] (alpha) and gv [B, H, L, d_v] (beta).
    Returns (o, s_final) as float64 arrays."""
    q, k, v, g, s0, _, (B, H, L, dk, dv) = _prepare(q, k, v, g, "keydim", s0)
    gv = _f64(gv)
    if gv is None or gv.shape != (B, H, L, dv):
        raise ValueError("oracle: gv must be [B,H,L,d_v]")
    o = np.zeros((B, H, L, dv), dtype=np.float64)
    s = np.zeros((B, H, dk, dv), dtype=np.float64)
    nthreads = default_threads() if nthreads is None else int(nthreads)
    rc = _load(lib_path).gla_oracle_forward_outer(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gv),
                                                  FEATURE_MAPS[feature_map], _ptr(s0), _ptr(o), _ptr(s),
                                                  B, H, L, dk, dv, nthreads)
    if rc != 0:
        raise RuntimeError("gla_oracle_forward_outer failed with code %d" % rc)
    return o, s
