"""The pins must be able to see a plausible mistake in the oracle.

Each case plants one mistake in a private copy of ``oracle/recurrence.py``
(by a source-text substitution, CPU only), swaps the copy in for the real
oracle inside the pin module, and requires that at least one pin fails.
"""

import inspect
import types

import numpy as np
import pytest

import oracle.recurrence as rec
import tests.test_oracle_pins as pins

SRC = inspect.getsource(rec)

MUTANTS = {
    # decay applied after the prediction instead of before it
    "forget_after_predict": [
        ("            # forget\n            if decay == \"scalar\":\n                S *= np.exp(gf[sl, t])[:, None, None]\n            elif decay == \"channel\":\n                S *= np.exp(gf[sl, t])[:, :, None]\n", ""),
        ("            r = np.matmul(e[:, None, :], S)[:, 0, :]\n",
         "            r = np.matmul(e[:, None, :], S)[:, 0, :]\n"
         "            if decay == \"scalar\":\n                S *= np.exp(gf[sl, t])[:, None, None]\n"
         "            elif decay == \"channel\":\n                S *= np.exp(gf[sl, t])[:, :, None]\n"),
    ],
    # read the state before the write
    "read_before_write": [
        ("            S += kt[:, :, None] * (z - r)[:, None, :]\n            # read the post-update state\n            o[sl, t] = np.matmul(qf[sl, t][:, None, :], S)[:, 0, :]\n",
         "            o[sl, t] = np.matmul(qf[sl, t][:, None, :], S)[:, 0, :]\n            S += kt[:, :, None] * (z - r)[:, None, :]\n"),
    ],
    # sign error in the correction
    "sign_error": [("(z - r)[:, None, :]", "(z + r)[:, None, :]")],
    # erase with k instead of e (drops the erase gate)
    "erase_gate_dropped": [("r = np.matmul(e[:, None, :], S)", "r = np.matmul(kt[:, None, :], S)")],
    # write gate dropped
    "write_gate_dropped": [("z = wf[sl, t] * vf[sl, t]", "z = vf[sl, t]")],
    # per-channel decay applied to the value axis
    "decay_on_value_axis": [("S *= np.exp(gf[sl, t])[:, :, None]", "S *= np.exp(gf[sl, t]).mean(axis=1)[:, None, None]")],
    # query mixed into the write direction as well
    "qmix_in_write": [("S += kt[:, :, None] * (z - r)[:, None, :]",
                       "S += (kt + (lamf[sl, t, None] * qf[sl, t] if qmix else 0))[:, :, None] * (z - r)[:, None, :]")],
    # lambda ignored
    "lambda_ignored": [("x = kt + lamf[sl, t, None] * qf[sl, t] if qmix else kt", "x = kt")],
    # lambda_t read one token late
    "lambda_t_shifted": [("x = kt + lamf[sl, t, None] * qf[sl, t] if qmix else kt",
                          "x = kt + lamf[sl, max(t - 1, 0), None] * qf[sl, t] if qmix else kt")],
    # per-value-channel beta applied to the write only, not to the prediction
    "value_beta_write_only": [("(bef[sl, t] * (vf[sl, t] - r))", "(bef[sl, t] * vf[sl, t] - r)")],
    # per-value-channel beta predicting before the decay
    "value_beta_decay_after_write": [
        ("            if erase == \"value\":\n", "            if erase == \"value\":\n                S /= np.exp(gf[sl, t])[:, None, None] if decay == \"scalar\" else 1.0\n")],
    # beta applied twice to the written value
    "beta_twice": [("z = bef[sl, t, None] * vf[sl, t]", "z = bef[sl, t, None] ** 2 * vf[sl, t]")],
    # readout along k instead of q
    "read_along_k": [("o[sl, t] = np.matmul(qf[sl, t][:, None, :], S)", "o[sl, t] = np.matmul(kf[sl, t][:, None, :], S)")],
    # state ignored (always starts from zero)
    "initial_state_ignored": [("S = S0[sl].copy()", "S = np.zeros_like(S0[sl])")],
}


def _mutant(edits):
    src = SRC
    for old, new in edits:
        assert old in src, f"mutation anchor not found: {old[:60]!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod.gdr_recurrence


def _pin_functions():
    fns = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if not params:
            fns.append((name, fn, {}))
            continue
        # expand the first value of every parametrize mark only (keeps it fast)
        kw = {}
        for m in params:
            names = [n.strip() for n in m.args[0].split(",")]
            vals = m.args[1][0] if len(names) > 1 else (m.args[1][0],)
            kw.update(dict(zip(names, vals)))
        fns.append((name, fn, kw))
    return fns


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_some_pin_fails_on_mutant(mutant, monkeypatch):
    bad = _mutant(MUTANTS[mutant])
    monkeypatch.setattr(pins, "gdr_recurrence", bad)
    failed = []
    for name, fn, kw in _pin_functions():
        try:
            with np.errstate(all="ignore"):
                fn(**kw)
        except Exception:  # AssertionError or a shape error both count as detection
            failed.append(name)
    assert failed, f"no pin detects the mutant {mutant}"


def test_unmutated_copy_passes_every_pin(monkeypatch):
    good = _mutant([])
    monkeypatch.setattr(pins, "gdr_recurrence", good)
    for name, fn, kw in _pin_functions():
        fn(**kw)
