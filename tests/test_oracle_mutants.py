"""CPU tests: the pins are strong enough to catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of ``oracle/gla_oracle.c`` (on the CPU, in a
temporary directory), builds it, and requires that at least one pin of ``pins.py``
rejects it.  The committed oracle itself must pass every pin (test_oracle_pins).
"""
import functools
import os

import pytest

from oracle import oracle
from tests import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "gla_oracle.c")

UPDATE = "S[i * dv + j] = a[i] * bv[j] * S[i * dv + j] + kf[i] * v[t * dv + j];"
READ = "acc += qf[i] * S[i * dv + j];"
DELTA_ERR = "z[j] = bt * (v[t * dv + j] - pred);"

MUTANTS = {
    "no_decay": [(UPDATE, "S[i * dv + j] = S[i * dv + j] + kf[i] * v[t * dv + j];")],
    "gate_sign": [("a[i] = exp(jb->g[(head * L + t) * dk + i]);",
                   "a[i] = exp(-jb->g[(head * L + t) * dk + i]);")],
    # the outer-product gate
    "outer_value_gate_ignored": [("bv[j] = jb->gate_mode == ORACLE_GATE_OUTER ? exp(jb->gv[(head * L + t) * dv + j]) : 1.0;",
                                  "bv[j] = 1.0;")],
    "outer_value_gate_sign": [("exp(jb->gv[(head * L + t) * dv + j])", "exp(-jb->gv[(head * L + t) * dv + j])")],
    "outer_value_gate_wrong_token": [("exp(jb->gv[(head * L + t) * dv + j])",
                                      "exp(jb->gv[(head * L + (t > 0 ? t - 1 : 0)) * dv + j])")],
    "outer_value_gate_key_index": [("exp(jb->gv[(head * L + t) * dv + j])",
                                    "exp(jb->gv[(head * L + t) * dv + (j % dk)])")],
    "outer_value_gate_on_write": [(UPDATE, "S[i * dv + j] = a[i] * S[i * dv + j] + bv[j] * kf[i] * v[t * dv + j];")],
    "decay_after_write": [(UPDATE, "S[i * dv + j] = a[i] * bv[j] * (S[i * dv + j] + kf[i] * v[t * dv + j]);")],
    "gate_on_value_axis": [(UPDATE, "S[i * dv + j] = a[j % dk] * bv[j] * S[i * dv + j] + kf[i] * v[t * dv + j];")],
    "wrong_readout_column": [(READ, "acc += qf[i] * S[i * dv + (dv - 1 - j)];")],
    "readout_uses_key": [(READ, "acc += kf[i] * S[i * dv + j];")],
    "phi_on_value": [(UPDATE, "S[i * dv + j] = a[i] * bv[j] * S[i * dv + j] + kf[i] * feature(v[t * dv + j], jb->phi);")],
    "phi_missing_on_query": [("qf[i] = feature(q[t * dk + i], jb->phi);", "qf[i] = q[t * dk + i];")],
    "elu_without_plus_one": [("return x > 0.0 ? x + 1.0 : exp(x);", "return x > 0.0 ? x : exp(x);")],
    "scalar_gate_head_offset": [("a[i] = exp(jb->g[head * L + t]);", "a[i] = exp(jb->g[t]);")],
    "initial_state_ignored": [("if (jb->s0) memcpy", "if (0) memcpy")],
    "exclusive_readout": [
        ("""        /* state update: decay the key rows (and value columns), then add k~ v^T */
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                S[i * dv + j] = a[i] * bv[j] * S[i * dv + j] + kf[i] * v[t * dv + j];
""", ""),
        ("""            o[t * dv + j] = jb->norm ? acc / den : acc;
        }""", """            o[t * dv + j] = jb->norm ? acc / den : acc;
        }
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                S[i * dv + j] = a[i] * bv[j] * S[i * dv + j] + kf[i] * v[t * dv + j];""")],
    "off_by_one_value_row": [(UPDATE, "S[i * dv + j] = a[i] * bv[j] * S[i * dv + j] + kf[i] * v[(t > 0 ? t - 1 : 0) * dv + j];")],
    # the normalised form
    "norm_z_no_decay": [("z[i] = a[i] * z[i] + kf[i];", "z[i] = z[i] + kf[i];")],
    "norm_den_uses_key": [("den += qf[i] * z[i];", "den += kf[i] * z[i];")],
    "norm_exclusive_den": [("""                z[i] = a[i] * z[i] + kf[i];
                den += qf[i] * z[i];""", """                den += qf[i] * z[i];
                z[i] = a[i] * z[i] + kf[i];""")],
    "norm_z0_ignored": [("if (jb->z0) memcpy", "if (0) memcpy")],
    "norm_not_divided": [("o[t * dv + j] = jb->norm ? acc / den : acc;", "o[t * dv + j] = acc;")],
    "norm_z_value_weighted": [("z[i] = a[i] * z[i] + kf[i];", "z[i] = a[i] * z[i] + kf[i] * v[t * dv];")],
    # the delta rule
    "delta_no_strength": [(DELTA_ERR, "z[j] = (v[t * dv + j] - pred);")],
    "delta_error_sign": [(DELTA_ERR, "z[j] = bt * (v[t * dv + j] + pred);")],
    "delta_no_prediction": [(DELTA_ERR, "z[j] = bt * v[t * dv + j];")],
    "delta_predicts_with_query": [("pred += k[t * dk + i] * S[i * dv + j];", "pred += q[t * dk + i] * S[i * dv + j];")],
    "delta_strength_head_offset": [("const double bt = jb->beta[head * L + t];", "const double bt = jb->beta[t];")],
    "delta_write_unscaled_key": [("S[i * dv + j] += k[t * dk + i] * z[j];", "S[i * dv + j] += z[j];")],
    "delta_exclusive_readout": [
        ("""        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j) S[i * dv + j] += k[t * dk + i] * z[j];
""", ""),
        ("""            o[t * dv + j] = acc;
        }
    }""", """            o[t * dv + j] = acc;
        }
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j) S[i * dv + j] += k[t * dk + i] * z[j];
    }""")],
}


def _pin_results(fwd, fwd_norm, fwd_delta, fwd_outer):
    failed = []
    for name, (fn, tol) in pins.OUTER_ERROR_PINS.items():
        try:
            err = fn(fwd_outer)
        except AssertionError:
            failed.append(name)
            continue
        if not err <= tol:
            failed.append(name)
    for name, (fn, tol) in pins.DELTA_ERROR_PINS.items():
        try:
            err = fn(fwd_delta)
        except AssertionError:
            failed.append(name)
            continue
        if not err <= tol:
            failed.append(name)
    for name, (fn, tol) in pins.NORM_ERROR_PINS.items():
        try:
            err = fn(fwd_norm)
        except AssertionError:
            failed.append(name)
            continue
        if not err <= tol:
            failed.append(name)
    for name, (fn, tol) in pins.ALL_ERROR_PINS.items():
        try:
            err = fn(fwd)
        except AssertionError:
            failed.append(name)
            continue
        if not err <= tol:                 # also catches NaN
            failed.append(name)
    try:
        if not pins.pin_positive_monotone(fwd) > 0.0:
            failed.append("positive_monotone")
    except AssertionError:
        failed.append("positive_monotone")
    return failed


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_reject_planted_mistake(mutant, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[mutant]:
        assert src.count(old) == 1, "mutation anchor not found: %r" % old
        src = src.replace(old, new)
    c_path = tmp_path / ("mutant_%s.c" % mutant)
    c_path.write_text(src)
    lib = oracle.compile_source(str(c_path), str(tmp_path / ("libmutant_%s.so" % mutant)))
    fwd = functools.partial(oracle.forward, lib_path=lib)
    fwd_norm = functools.partial(oracle.forward_norm, lib_path=lib)
    fwd_delta = functools.partial(oracle.forward_delta, lib_path=lib)
    fwd_outer = functools.partial(oracle.forward_outer, lib_path=lib)
    failed = _pin_results(fwd, fwd_norm, fwd_delta, fwd_outer)
    assert failed, "planted mistake %r passed every pin" % mutant
