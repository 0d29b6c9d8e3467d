"""fp64 CPU oracle of the causal gated-linear-attention forward pass.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py``; never by the product package.
"""
