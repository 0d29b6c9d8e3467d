"""Causal gated linear attention (GLA) forward for AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
``include/gla.h`` (``libgla.so``, built in-tree); this package is its thin Python
binding.  ``inputs`` holds the seeded synthetic workloads.
"""
from .api import (DeviceState, decode_step, decode_step_delta, decode_step_norm,  # noqa: F401
                  decode_step_outer, delta_workspace_bytes, gate_project, prefill, prefill_delta,
                  prefill_norm, prefill_outer, state_alloc, workspace_bytes)
from ._lib import GLAError  # noqa: F401
