"""Plant plausible mistakes in a copy of the C oracle and check that the pins
catch every one of them.  The mutants are compiled from edited copies of the
source into a temporary directory; the oracle itself is never modified."""
import os
import subprocess

import pytest

import oracle
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "hgrn2_oracle.c")

# (name, text to replace, replacement)
MUTANTS = [
    ("no_decay", "row[j] = f * row[j] + k[c] * v[j];", "row[j] = row[j] + k[c] * v[j];"),
    ("decay_after_write", "row[j] = f * row[j] + k[c] * v[j];", "row[j] = f * (row[j] + k[c] * v[j]);"),
    ("readout_before_update",
     "      step_state(DK, DV, S, k + tok_off(T, H, DK, b, t, h), v + tok_off(T, H, DV, b, t, h),\n"
     "                 log_f + tok_off(T, H, DK, b, t, h));\n"
     "      readout(DK, DV, S, q + tok_off(T, H, DK, b, t, h), y + tok_off(T, H, DV, b, t, h));",
     "      readout(DK, DV, S, q + tok_off(T, H, DK, b, t, h), y + tok_off(T, H, DV, b, t, h));\n"
     "      step_state(DK, DV, S, k + tok_off(T, H, DK, b, t, h), v + tok_off(T, H, DV, b, t, h),\n"
     "                 log_f + tok_off(T, H, DK, b, t, h));"),
    ("readout_transposed", "for (int j = 0; j < DV; ++j) y[j] += q[c] * row[j];",
     "for (int j = 0; j < DV; ++j) y[j] += q[j % DK] * S[(size_t)(j % DK) * DV + (c % DV)];"),
    ("decay_on_columns", "const double f = exp(log_f[c]);\n    double *row = S + (size_t)c * DV;\n    for (int j = 0; j < DV; ++j) row[j] = f * row[j] + k[c] * v[j];",
     "double *row = S + (size_t)c * DV;\n    for (int j = 0; j < DV; ++j) row[j] = exp(log_f[j % DK]) * row[j] + k[c] * v[j];"),
    ("h0_ignored", "if (h0) memcpy(S, h0 + (size_t)bh * SS, SS * sizeof(double));\n    else memset(S, 0, SS * sizeof(double));\n    for (int t = 0; t < T; ++t) {\n      step_state",
     "memset(S, 0, SS * sizeof(double));\n    for (int t = 0; t < T; ++t) {\n      step_state"),
    ("bwd_missing_f_factor", "gl[c] = exp(lt[c]) * al;", "gl[c] = al;"),
    ("bwd_wrong_state", "al += G[(size_t)c * DV + j] * Sp[(size_t)c * DV + j];",
     "al += G[(size_t)c * DV + j] * St[(size_t)c * DV + j];"),
    ("bwd_q_for_k", "G[(size_t)c * DV + j] += qt[c] * gy[j];", "G[(size_t)c * DV + j] += kt[c] * gy[j];"),
    ("bwd_dq_prev_state", "aq += St[(size_t)c * DV + j] * gy[j];", "aq += Sp[(size_t)c * DV + j] * gy[j];"),
    ("bwd_no_adjoint_decay", "for (int j = 0; j < DV; ++j) G[(size_t)c * DV + j] *= f;",
     "for (int j = 0; j < DV; ++j) G[(size_t)c * DV + j] *= 1.0;"),
    ("bwd_dk_before_accumulate",
     "        for (int c = 0; c < DK; ++c)\n          for (int j = 0; j < DV; ++j) G[(size_t)c * DV + j] += qt[c] * gy[j];\n",
     ""),
    ("decode_readout_first",
     "    step_state(DK, DV, S, k + (size_t)bh * DK, v + (size_t)bh * DV, log_f + (size_t)bh * DK);\n    readout(DK, DV, S, q + (size_t)bh * DK, y + (size_t)bh * DV);",
     "    readout(DK, DV, S, q + (size_t)bh * DK, y + (size_t)bh * DV);\n    step_state(DK, DV, S, k + (size_t)bh * DK, v + (size_t)bh * DV, log_f + (size_t)bh * DK);"),
    ("checkpoint_off_by_one", "if (t % ORACLE_CKPT == 0) memcpy", "if (t % ORACLE_CKPT == 1) memcpy"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, name
    mutated = src.replace(old, new, 1)
    assert mutated != src
    c = tmp_path / (name + ".c")
    c.write_text(mutated)
    so = tmp_path / ("lib" + name + ".so")
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", str(c),
                           "-o", str(so), "-lm"])
    return oracle.Oracle(str(so))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    orc = _build_mutant(tmp_path, name, old, new)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
        except Exception as e:  # a crash or NaN also counts as detected
            caught.append(pin.__name__ + ":" + type(e).__name__)
    assert caught, "mutant %s passed every pin" % name


# Plausible mistakes in the gate-mode chain rule and gate formula of the
# oracle (its Python part); each replaces one oracle function for the duration
# of the test and must fail at least one gate pin.
def _gate_mutants():
    import numpy as np
    o = oracle
    good_p, good_l, good_k = o.gate_partials, o.gate_log_f, o.gate_k

    def no_inv_f(z, lam):
        a, b, c, d = good_p(z, lam)
        f = np.exp(good_l(z, lam))
        return a * f, b, c * f, d

    def dk_dz_sign(z, lam):
        a, b, c, d = good_p(z, lam)
        return a, -b, c, d

    def dlam_from_dz(z, lam):
        a, b, c, d = good_p(z, lam)
        return a, b, a, b

    def no_one_minus_lam(z, lam):
        a, b, c, d = good_p(z, lam)
        lam = np.asarray(lam, dtype=np.float64)
        return a / (1.0 - lam), b / (1.0 - lam), c, d

    def logf_no_lam(z, lam):
        return good_l(z, 0.0 * np.asarray(lam))

    def k_untied(z, lam):
        return good_k(z, 0.0 * np.asarray(lam))

    return [("gate_partials", no_inv_f), ("gate_partials", dk_dz_sign), ("gate_partials", dlam_from_dz),
            ("gate_partials", no_one_minus_lam), ("gate_log_f", logf_no_lam), ("gate_k", k_untied)]


@pytest.mark.parametrize("which", range(6))
def test_gate_pins_catch_mutant(which, monkeypatch):
    name, fn = _gate_mutants()[which]
    monkeypatch.setattr(oracle, name, fn)
    orc = oracle.default()
    caught = []
    for pin in pins.GATE_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "gate mutant %d (%s) passed every gate pin" % (which, name)
