"""CPU tests of the gate producer's oracle (``oracle/gate_oracle.py``): it passes
every pin of ``pins.GATE_ERROR_PINS``, and each planted mistake (in a copy of its
source, loaded from a temporary file) fails at least one of them."""
import importlib.util
import os

import numpy as np
import pytest

from oracle import gate_oracle
from tests import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "gate_oracle.py")


@pytest.mark.parametrize("name", sorted(pins.GATE_ERROR_PINS))
def test_gate_oracle_pin(name):
    fn, tol = pins.GATE_ERROR_PINS[name]
    err = fn(gate_oracle.gate_project)
    assert err <= tol, "%s: error %.3e above %.1e" % (name, err, tol)


def test_gate_oracle_rejects_bad_shapes():
    x, wd, wu = np.zeros((1, 2, 8)), np.zeros((4, 8)), np.zeros((6, 4))
    with pytest.raises(ValueError):
        gate_oracle.gate_project(x, wd, wu, 2, 4)           # H * d_k = 8 rows expected


MUTANTS = {
    "sigmoid_not_log": ("g = -np.logaddexp(0.0, -z) / float(tau)", "g = 1.0 / (1.0 + np.exp(-z)) / float(tau)"),
    "log_one_minus_sigmoid": ("g = -np.logaddexp(0.0, -z) / float(tau)", "g = -np.logaddexp(0.0, z) / float(tau)"),
    "tau_multiplies": ("g = -np.logaddexp(0.0, -z) / float(tau)", "g = -np.logaddexp(0.0, -z) * float(tau)"),
    "rank_slots_reversed": ("zd = x @ w_down.T", "zd = x @ w_down[::-1].T"),
    "layout_not_transposed": ("g.reshape(B, L, H, d_k).transpose(0, 2, 1, 3)", "g.reshape(B, H, L, d_k)"),
    "head_and_dim_swapped": ("g.reshape(B, L, H, d_k).transpose(0, 2, 1, 3)",
                             "g.reshape(B, L, d_k, H).transpose(0, 3, 1, 2)"),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_gate_pins_reject_planted_mistake(mutant, tmp_path):
    old, new = MUTANTS[mutant]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not found: %r" % old
    path = tmp_path / ("gate_mutant_%s.py" % mutant)
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("gate_mutant_%s" % mutant, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = []
    for name, (fn, tol) in pins.GATE_ERROR_PINS.items():
        try:
            with np.errstate(all="ignore"):
                err = fn(mod.gate_project)
        except (AssertionError, ValueError):
            failed.append(name)
            continue
        if not err <= tol:
            failed.append(name)
    assert failed, "planted mistake %r passed every pin" % mutant
