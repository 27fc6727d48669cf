"""The fp64 row-softmax oracle against its pins, and planted mistakes in
copies of it (each must fail at least one pin)."""
import os

import numpy as np
import pytest

import oracle
import softmax_pins

SRC = os.path.join(os.path.dirname(os.path.abspath(oracle.__file__)), "softmax.py")


@pytest.mark.parametrize("check", softmax_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_softmax_oracle_pin(check):
    check(oracle.row_softmax)


MUTANTS = {
    "no_max_subtraction": [("e = np.exp(row - m)", "e = np.exp(row)")],
    "no_normalisation": [("y[i] = e / l", "y[i] = e")],
    "sum_of_inputs": [("l = e.sum()", "l = row.sum()")],
    "min_instead_of_max": [("m = row.max()", "m = row.min()")],
    "global_max": [("m = row.max()", "m = x.max()")],
    "last_column_dropped": [("l = e.sum()", "l = e[:-1].sum() if N > 1 else e.sum()")],
    "wrong_sign": [("e = np.exp(row - m)", "e = np.exp(m - row)")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert old in src, "mutation anchor missing: %r" % old
        src = src.replace(old, new, 1)
    ns = {}
    exec(compile(src, str(tmp_path / "mutant.py"), "exec"), ns)
    failed = []
    with np.errstate(all="ignore"):
        for check in softmax_pins.ALL_CHECKS:
            try:
                check(ns["row_softmax"])
            except AssertionError:
                failed.append(check.__name__)
                break
    assert failed, "planted mistake %r passed every pin" % name
