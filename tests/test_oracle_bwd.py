"""The fp64 backward oracle against facts fixed by the pages and by mathematics.

Every check lives in ``oracle_bwd_pins.py`` so that
``test_oracle_bwd_mutants.py`` can run the same checks against copies of the
oracle with a planted mistake.
"""
import numpy as np
import pytest

import oracle
import oracle_bwd_pins


def _grads(q, k, v, dout, causal, scale, qrows=None, krows=None):
    return oracle.attn_bwd_oracle(q, k, v, dout, causal=causal, scale=scale, qrows=qrows,
                                  krows=krows)


@pytest.mark.parametrize("check", oracle_bwd_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_bwd_oracle_pin(check):
    check(_grads)


def test_bwd_oracle_rejects_bad_rows():
    q = np.zeros((1, 1, 4, 2))
    with pytest.raises(RuntimeError):
        oracle.attn_bwd_oracle(q, q, q, q, qrows=[4])
    with pytest.raises(RuntimeError):
        oracle.attn_bwd_oracle(q, q, q, q, krows=[-1])


def test_bwd_oracle_empty_row_lists():
    q = np.random.default_rng(0).standard_normal((1, 2, 6, 3))
    dq, dk, dv = oracle.attn_bwd_oracle(q, q, q, q, qrows=[], krows=[])
    assert dq.shape == (0, 3) and dk.shape == (0, 3) and dv.shape == (0, 3)
