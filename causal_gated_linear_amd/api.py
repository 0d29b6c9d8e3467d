"""Thin Python binding of the C ABI (include/gla.h): argument marshalling only.

PyTorch supplies device memory and the stream; every step of the computation runs
in the HIP kernels of ``libgla.so``.  Shapes are checked here because the C ABI
receives bare pointers and cannot see buffer sizes.

    o, s_final = prefill(q, k, v, log_gate=g, gate="keydim", chunk=64)
    o = decode_step(q_t, k_t, v_t, log_gate=g_t, state=s, gate="keydim")   # s updated
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.GLA_F32, torch.bfloat16: _lib.GLA_BF16}


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_tensor(t, name, shape, dtype, device):
    _need(isinstance(t, torch.Tensor), "%s must be a tensor" % name)
    _need(tuple(t.shape) == tuple(shape), "%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    _need(t.dtype == dtype, "%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    _need(t.is_contiguous(), "%s must be contiguous" % name)
    _need(t.device == device, "%s is on %s, expected %s" % (name, t.device, device))


def _workspace(nbytes, dev, stream):
    """A device workspace of nbytes for a launch on ``stream``.  The tensor is freed when
    the caller returns, while the kernel may still run: record the launch stream, so
    the caching allocator reuses the memory only after the work queued there."""
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if stream is not None:
        ws.record_stream(stream)
    return ws


def workspace_bytes(B, H, L, d_k, d_v, chunk, dtype=torch.bfloat16) -> int:
    """Bytes of device workspace gla_prefill_chunked needs for these sizes."""
    return int(_lib.load().gla_prefill_workspace_bytes(B, H, L, d_k, d_v, chunk, _DTYPES[dtype]))


def _check_prefill(q, k, v, log_gate, gate, initial_state):
    _need(q.dim() == 4 and v.dim() == 4, "q, k, v must be 4-D [B, H, L, d]")
    B, H, L, dk = q.shape
    dv = v.shape[3]
    dev, dt = q.device, q.dtype
    _need(dt in _DTYPES, "dtype must be float32 or bfloat16")
    _check_tensor(q, "q", (B, H, L, dk), dt, dev)
    _check_tensor(k, "k", (B, H, L, dk), dt, dev)
    _check_tensor(v, "v", (B, H, L, dv), dt, dev)
    gate = gate if gate is not None else (None if log_gate is None else "keydim")
    _need(gate in _lib.GATES, "gate must be None, 'keydim' or 'scalar'")
    if gate == "keydim":
        _check_tensor(log_gate, "log_gate", (B, H, L, dk), torch.float32, dev)
    elif gate == "scalar":
        _check_tensor(log_gate, "log_gate", (B, H, L), torch.float32, dev)
    else:
        _need(log_gate is None, "log_gate given without a gate mode")
    if initial_state is not None:
        _check_tensor(initial_state, "initial_state", (B, H, dk, dv), torch.float32, dev)
    _need(dev.type == "cuda", "tensors must be on a GPU device")
    return B, H, L, dk, dv, dev, dt, gate


def prefill(q, k, v, log_gate=None, gate=None, initial_state=None, chunk=64, feature_map=None,
            out=None, final_state=None, workspace=None, stream=None):
    """Chunkwise GLA prefill (gla_prefill_chunked).

    q, k: [B, H, L, d_k]; v: [B, H, L, d_v] (fp32 or bf16, same dtype, CUDA);
    log_gate: fp32 [B, H, L, d_k] (gate="keydim") or [B, H, L] (gate="scalar");
    initial_state: fp32 [B, H, d_k, d_v] or None.  Returns (o, s_final).
    ``final_state`` may be ``initial_state`` to update it in place.
    """
    lib = _lib.load()
    B, H, L, dk, dv, dev, dt, gate = _check_prefill(q, k, v, log_gate, gate, initial_state)
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=dt, device=dev)
    else:
        _check_tensor(out, "out", (B, H, L, dv), dt, dev)
    if final_state is None:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    else:
        _check_tensor(final_state, "final_state", (B, H, dk, dv), torch.float32, dev)
    need = workspace_bytes(B, H, L, dk, dv, chunk, dt)
    if need and workspace is None:
        workspace = _workspace(need, dev, stream)
    if workspace is not None:
        _need(workspace.is_contiguous() and workspace.device == dev, "workspace must be contiguous on %s" % dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gla_prefill_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(log_gate), _lib.GATES[gate],
                                 _ptr(initial_state), _ptr(out), _ptr(final_state),
                                 B, H, L, dk, dv, int(chunk), _DTYPES[dt],
                                 _lib.FEATURE_MAPS[feature_map], _ptr(workspace), ws_bytes,
                                 _stream_handle(stream))
    _lib.check(st, "gla_prefill_chunked")
    return out, final_state


def prefill_noalloc(q, k, v, log_gate=None, gate=None, initial_state=None, chunk=64, feature_map=None,
                    out=None, final_state=None, stream=None):
    """gla_prefill_chunked_noalloc: ``prefill`` without a workspace; the library's own
    per-GPU scratch array serves segmented sizes (at most 32 MiB of workspace).  The
    C entry point allocates nothing; pass ``out`` and ``final_state`` to keep this
    wrapper from allocating them.  Returns (o, s_final)."""
    lib = _lib.load()
    B, H, L, dk, dv, dev, dt, gate = _check_prefill(q, k, v, log_gate, gate, initial_state)
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=dt, device=dev)
    else:
        _check_tensor(out, "out", (B, H, L, dv), dt, dev)
    if final_state is None:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    else:
        _check_tensor(final_state, "final_state", (B, H, dk, dv), torch.float32, dev)
    st = lib.gla_prefill_chunked_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_gate), _lib.GATES[gate],
                                         _ptr(initial_state), _ptr(out), _ptr(final_state), B, H, L, dk, dv,
                                         int(chunk), _DTYPES[dt], _lib.FEATURE_MAPS[feature_map],
                                         _stream_handle(stream))
    _lib.check(st, "gla_prefill_chunked_noalloc")
    return out, final_state


def prefill_norm(q, k, v, log_gate=None, gate=None, initial_state=None, initial_norm=None, chunk=64,
                 feature_map=None, out=None, final_state=None, final_norm=None, stream=None):
    """Normalised chunkwise prefill (gla_prefill_chunked_norm): as ``prefill``, with the
    normaliser state z (fp32 [B, H, d_k]); o_t = S_t^T phi(q_t) / phi(q_t) . z_t.
    Returns (o, s_final, z_final); ``final_state`` may be ``initial_state`` (in place),
    ``final_norm`` must be a buffer of its own."""
    lib = _lib.load()
    B, H, L, dk, dv, dev, dt, gate = _check_prefill(q, k, v, log_gate, gate, initial_state)
    if initial_norm is not None:
        _check_tensor(initial_norm, "initial_norm", (B, H, dk), torch.float32, dev)
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=dt, device=dev)
    else:
        _check_tensor(out, "out", (B, H, L, dv), dt, dev)
    if final_state is None:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    else:
        _check_tensor(final_state, "final_state", (B, H, dk, dv), torch.float32, dev)
    if final_norm is None:
        final_norm = torch.empty((B, H, dk), dtype=torch.float32, device=dev)
    else:
        _check_tensor(final_norm, "final_norm", (B, H, dk), torch.float32, dev)
    st = lib.gla_prefill_chunked_norm(_ptr(q), _ptr(k), _ptr(v), _ptr(log_gate), _lib.GATES[gate],
                                      _ptr(initial_state), _ptr(initial_norm), _ptr(out),
                                      _ptr(final_state), _ptr(final_norm), B, H, L, dk, dv, int(chunk),
                                      _DTYPES[dt], _lib.FEATURE_MAPS[feature_map], _stream_handle(stream))
    _lib.check(st, "gla_prefill_chunked_norm")
    return out, final_state, final_norm


def _check_decode(q, k, v, log_gate, gate, state, out):
    _need(q.dim() == 3 and v.dim() == 3, "q, k, v must be 3-D [B, H, d]")
    B, H, dk = q.shape
    dv = v.shape[2]
    dev, dt = q.device, q.dtype
    _need(dt in _DTYPES, "dtype must be float32 or bfloat16")
    _check_tensor(q, "q", (B, H, dk), dt, dev)
    _check_tensor(k, "k", (B, H, dk), dt, dev)
    _check_tensor(v, "v", (B, H, dv), dt, dev)
    gate = gate if gate is not None else (None if log_gate is None else "keydim")
    _need(gate in _lib.GATES, "gate must be None, 'keydim' or 'scalar'")
    if gate == "keydim":
        _check_tensor(log_gate, "log_gate", (B, H, dk), torch.float32, dev)
    elif gate == "scalar":
        _check_tensor(log_gate, "log_gate", (B, H), torch.float32, dev)
    else:
        _need(log_gate is None, "log_gate given without a gate mode")
    _need(state is not None, "state is required")
    _check_tensor(state, "state", (B, H, dk, dv), torch.float32, dev)
    _need(dev.type == "cuda", "tensors must be on a GPU device")
    if out is None:
        out = torch.empty((B, H, dv), dtype=dt, device=dev)
    else:
        _check_tensor(out, "out", (B, H, dv), dt, dev)
    return B, H, dk, dv, dev, dt, gate, out


def decode_step(q, k, v, log_gate=None, state=None, gate=None, feature_map=None, out=None,
                stream=None):
    """One recurrent step (gla_decode_step); ``state`` [B, H, d_k, d_v] fp32 is updated
    in place.  q, k: [B, H, d_k]; v: [B, H, d_v]; log_gate: fp32 [B, H, d_k] (keydim)
    or [B, H] (scalar).  Returns o [B, H, d_v]."""
    lib = _lib.load()
    B, H, dk, dv, dev, dt, gate, out = _check_decode(q, k, v, log_gate, gate, state, out)
    st = lib.gla_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_gate), _lib.GATES[gate],
                             _ptr(state), _ptr(out), B, H, dk, dv, _DTYPES[dt],
                             _lib.FEATURE_MAPS[feature_map], _stream_handle(stream))
    _lib.check(st, "gla_decode_step")
    return out


def decode_step_norm(q, k, v, log_gate=None, state=None, norm=None, gate=None, feature_map=None,
                     out=None, stream=None):
    """One step of the normalised recurrence (gla_decode_step_norm); ``state`` and the
    normaliser state ``norm`` (fp32 [B, H, d_k]) are updated in place.  Returns o."""
    lib = _lib.load()
    B, H, dk, dv, dev, dt, gate, out = _check_decode(q, k, v, log_gate, gate, state, out)
    _need(norm is not None, "norm (the normaliser state) is required")
    _check_tensor(norm, "norm", (B, H, dk), torch.float32, dev)
    st = lib.gla_decode_step_norm(_ptr(q), _ptr(k), _ptr(v), _ptr(log_gate), _lib.GATES[gate],
                                  _ptr(state), _ptr(norm), _ptr(out), B, H, dk, dv, _DTYPES[dt],
                                  _lib.FEATURE_MAPS[feature_map], _stream_handle(stream))
    _lib.check(st, "gla_decode_step_norm")
    return out


def delta_workspace_bytes(B, H, L, d_k, d_v, chunk, dtype=torch.bfloat16) -> int:
    """Bytes of device workspace gla_prefill_delta needs for these sizes."""
    return int(_lib.load().gla_delta_workspace_bytes(B, H, L, d_k, d_v, chunk, _DTYPES[dtype]))


def prefill_delta(q, k, v, beta, initial_state=None, chunk=32, out=None, final_state=None,
                  workspace=None, stream=None):
    """Chunkwise delta-rule prefill (gla_prefill_delta).

    q, k: [B, H, L, d_k]; v: [B, H, L, d_v] (fp32 or bf16, same dtype, CUDA);
    beta: fp32 [B, H, L] write strengths; initial_state: fp32 [B, H, d_k, d_v] or None.
    Returns (o, s_final); ``final_state`` may be ``initial_state`` to update it in place.
    """
    lib = _lib.load()
    B, H, L, dk, dv, dev, dt, _ = _check_prefill(q, k, v, None, None, initial_state)
    _check_tensor(beta, "beta", (B, H, L), torch.float32, dev)
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=dt, device=dev)
    else:
        _check_tensor(out, "out", (B, H, L, dv), dt, dev)
    if final_state is None:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    else:
        _check_tensor(final_state, "final_state", (B, H, dk, dv), torch.float32, dev)
    need = delta_workspace_bytes(B, H, L, dk, dv, chunk, dt)
    if need and workspace is None:
        workspace = _workspace(need, dev, stream)
    if workspace is not None:
        _need(workspace.is_contiguous() and workspace.device == dev, "workspace must be contiguous on %s" % dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gla_prefill_delta(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(initial_state), _ptr(out),
                               _ptr(final_state), B, H, L, dk, dv, int(chunk), _DTYPES[dt],
                               _ptr(workspace), ws_bytes, _stream_handle(stream))
    _lib.check(st, "gla_prefill_delta")
    return out, final_state


def decode_step_delta(q, k, v, beta, state=None, out=None, stream=None):
    """One delta-rule step (gla_decode_step_delta); ``state`` [B, H, d_k, d_v] fp32 is
    updated in place.  q, k: [B, H, d_k]; v: [B, H, d_v]; beta: fp32 [B, H].  Returns o."""
    lib = _lib.load()
    B, H, dk, dv, dev, dt, _, out = _check_decode(q, k, v, None, None, state, out)
    _check_tensor(beta, "beta", (B, H), torch.float32, dev)
    st = lib.gla_decode_step_delta(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(state), _ptr(out),
                                   B, H, dk, dv, _DTYPES[dt], _stream_handle(stream))
    _lib.check(st, "gla_decode_step_delta")
    return out


def gate_project(x, w_down, w_up, H, d_k, tau=1.0, out=None, stream=None):
    """Input-side gate producer (gla_gate_project): fp32 log-gates
    g [B, H, L, d_k] = log(sigmoid(W_up W_down x)) / tau for the key-dim prefill.
    x: [B, L, d_model]; w_down: [rank, d_model]; w_up: [H*d_k, rank] (fp32 or bf16,
    same dtype, CUDA)."""
    lib = _lib.load()
    _need(x.dim() == 3, "x must be 3-D [B, L, d_model]")
    B, L, dm = x.shape
    dev, dt = x.device, x.dtype
    _need(dt in _DTYPES, "dtype must be float32 or bfloat16")
    _need(w_down.dim() == 2, "w_down must be 2-D [rank, d_model]")
    r = w_down.shape[0]
    _check_tensor(x, "x", (B, L, dm), dt, dev)
    _check_tensor(w_down, "w_down", (r, dm), dt, dev)
    _check_tensor(w_up, "w_up", (H * d_k, r), dt, dev)
    _need(dev.type == "cuda", "tensors must be on a GPU device")
    if out is None:
        out = torch.empty((B, H, L, d_k), dtype=torch.float32, device=dev)
    else:
        _check_tensor(out, "out", (B, H, L, d_k), torch.float32, dev)
    st = lib.gla_gate_project(_ptr(x), _ptr(w_down), _ptr(w_up), _ptr(out), B, L, dm, r, H, d_k, float(tau),
                              _DTYPES[dt], _stream_handle(stream))
    _lib.check(st, "gla_gate_project")
    return out


def prefill_outer(q, k, v, log_gate, log_gate_v, initial_state=None, chunk=64, feature_map=None, out=None,
                  final_state=None, stream=None):
    """Prefill with the outer-product gate G_t = alpha_t beta_t^T (gla_prefill_outer).

    q, k: [B, H, L, d_k]; v: [B, H, L, d_v]; log_gate: fp32 [B, H, L, d_k] (alpha);
    log_gate_v: fp32 [B, H, L, d_v] (beta); initial_state: fp32 [B, H, d_k, d_v] or None.
    Returns (o, s_final); ``final_state`` may be ``initial_state`` to update it in place.
    """
    lib = _lib.load()
    B, H, L, dk, dv, dev, dt, _ = _check_prefill(q, k, v, log_gate, "keydim", initial_state)
    _check_tensor(log_gate_v, "log_gate_v", (B, H, L, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=dt, device=dev)
    else:
        _check_tensor(out, "out", (B, H, L, dv), dt, dev)
    if final_state is None:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    else:
        _check_tensor(final_state, "final_state", (B, H, dk, dv), torch.float32, dev)
    st = lib.gla_prefill_outer(_ptr(q), _ptr(k), _ptr(v), _ptr(log_gate), _ptr(log_gate_v), _ptr(initial_state),
                               _ptr(out), _ptr(final_state), B, H, L, dk, dv, int(chunk), _DTYPES[dt],
                               _lib.FEATURE_MAPS[feature_map], _stream_handle(stream))
    _lib.check(st, "gla_prefill_outer")
    return out, final_state


def decode_step_outer(q, k, v, log_gate, log_gate_v, state=None, feature_map=None, out=None, stream=None):
    """One step with the outer-product gate (gla_decode_step_outer); ``state`` is updated
    in place.  log_gate: fp32 [B, H, d_k]; log_gate_v: fp32 [B, H, d_v].  Returns o."""
    lib = _lib.load()
    B, H, dk, dv, dev, dt, _, out = _check_decode(q, k, v, log_gate, "keydim", state, out)
    _check_tensor(log_gate_v, "log_gate_v", (B, H, dv), torch.float32, dev)
    st = lib.gla_decode_step_outer(_ptr(q), _ptr(k), _ptr(v), _ptr(log_gate), _ptr(log_gate_v), _ptr(state),
                                   _ptr(out), B, H, dk, dv, _DTYPES[dt], _lib.FEATURE_MAPS[feature_map],
                                   _stream_handle(stream))
    _lib.check(st, "gla_decode_step_outer")
    return out


class DeviceState:
    """A zeroed fp32 state [B, H, d_k, d_v] from gla_state_alloc, owned by this object
    (freed with gla_state_free).  ``tensor()`` views it as a torch tensor (no copy)
    through ``__cuda_array_interface__``; the view must not outlive the object."""

    def __init__(self, B, H, d_k, d_v, stream=None):
        lib = _lib.load()
        p = ctypes.c_void_p()
        _lib.check(lib.gla_state_alloc(B, H, d_k, d_v, ctypes.byref(p), _stream_handle(stream)),
                   "gla_state_alloc")
        self.ptr = p.value
        self.shape = (B, H, d_k, d_v)
        self._stream = stream

    @property
    def __cuda_array_interface__(self):
        return {"shape": self.shape, "typestr": "<f4", "data": (self.ptr, False), "version": 2,
                "strides": None}

    def tensor(self) -> torch.Tensor:
        return torch.as_tensor(self, device="cuda")

    def free(self):
        if self.ptr:
            _lib.check(_lib.load().gla_state_free(ctypes.c_void_p(self.ptr),
                                                  _stream_handle(self._stream)), "gla_state_free")
            self.ptr = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def state_alloc(B, H, d_k, d_v, stream=None) -> DeviceState:
    """gla_state_alloc: a zero-filled device state for decode_step."""
    return DeviceState(B, H, d_k, d_v, stream=stream)
