"""ctypes loader for ``libgla.so`` (the C ABI of include/gla.h).

The library must have been built in-tree (``python -m causal_gated_linear_amd.build``
or ``__graft_entry__.build()``); there is no fallback implementation, so a missing
library is a hard error.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgla.so")

# (name, restype, argtypes) for every entry point of include/gla.h and the test hook
# of include/gla_testing.h
_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
SIGNATURES = [
    ("gla_state_alloc", _I, [_I, _I, _I, _I, ctypes.POINTER(ctypes.c_void_p), _P]),
    ("gla_state_free", _I, [_P, _P]),
    ("gla_prefill_workspace_bytes", _SZ, [_I, _I, _I, _I, _I, _I, _I]),
    ("gla_prefill_chunked", _I, [_P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                 _P, _SZ, _P]),
    ("gla_prefill_chunked_noalloc", _I, [_P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P]),
    ("gla_decode_step", _I, [_P, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    ("gla_prefill_chunked_norm", _I, [_P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                      _I, _I, _I, _P]),
    ("gla_decode_step_norm", _I, [_P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    ("gla_delta_workspace_bytes", _SZ, [_I, _I, _I, _I, _I, _I, _I]),
    ("gla_prefill_delta", _I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _SZ, _P]),
    ("gla_decode_step_delta", _I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    ("gla_gate_project", _I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P]),
    ("gla_prefill_outer", _I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P]),
    ("gla_decode_step_outer", _I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    ("gla_strerror", ctypes.c_char_p, [_I]),
    ("gla_testing_set_plan", _I, [_I, _I, _I]),
    ("gla_last_error_detail", ctypes.c_char_p, []),
]

# gla_status values
GLA_OK = 0
GLA_ERR_NULL = -1
GLA_ERR_SHAPE = -2
GLA_ERR_UNSUPPORTED = -3
GLA_ERR_ALIGN = -4
GLA_ERR_ALIAS = -5
GLA_ERR_HIP = -6
GLA_ERR_OOM = -7
GLA_ERR_WORKSPACE = -8
# enums
GLA_F32, GLA_BF16 = 0, 1
GATES = {None: 0, "none": 0, "keydim": 1, "scalar": 2}
FEATURE_MAPS = {None: 0, "identity": 0, "elu1": 1}

_lib = None


class GLAError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__("%s failed (%d): %s" % (where, status, detail))


def load() -> ctypes.CDLL:
    """Load the in-tree ``libgla.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libgla.so is not built at %s; run `python -m "
                              "causal_gated_linear_amd.build` first" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int, where: str) -> None:
    if status != GLA_OK:
        lib = load()
        detail = (lib.gla_last_error_detail() or b"").decode()
        raise GLAError(status, where, detail or lib.gla_strerror(status).decode())
