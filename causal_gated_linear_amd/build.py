"""Builds ``libgla.so`` (the C ABI of include/gla.h plus its gfx950 kernels) in-tree.

hipcc compiles every HIP translation unit for gfx950 (in parallel; the prefill
kernel is instantiated per element type and d_k in separate units) and links the
shared library next to this file.  Run: ``python -m causal_gated_linear_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgla.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc")
CFLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
          # keep the compiler from emitting packed-fp32 VALU instructions
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _units():
    units = []
    for bf in (0, 1):
        for dk in (16, 32, 64, 128):
            units.append(("gla_prefill_inst.hip", "prefill_%d_%d.o" % (bf, dk),
                          ["-DGLA_INST_BF16=%d" % bf, "-DGLA_INST_DK=%d" % dk]))
    units.append(("gla_decode.hip", "decode.o", []))
    units.append(("gla_delta.hip", "delta.o", []))
    units.append(("gla_gate.hip", "gate.o", []))
    units.append(("gla_outer.hip", "outer.o", []))
    units.append(("gla_api.cpp", "api.o", ["-x", "hip"]))
    return units


def _compile(unit):
    src, obj, extra = unit
    out = os.path.join(BUILD, obj)
    cmd = [HIPCC] + CFLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (obj, "\n".join(msgs)))
    return out, msgs


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every unit and link ``libgla.so``; always rebuilds.  Returns its path."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found; cannot build the gfx950 kernels")
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(16, max(1, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, _units()))
    if verbose:
        for _, msgs in results:
            for m in msgs:
                print(m, file=sys.stderr)
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
