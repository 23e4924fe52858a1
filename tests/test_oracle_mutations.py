"""The hand-worked pins of H_X, the damping and the trace forms catch plausible mistakes in the oracle.

Each case plants one mistake in the oracle (on the CPU, for the duration of the test) and checks that
at least one of the hand-worked P18 pins then fails: dividing H_X = X^T X / n by n - 1 or not at all
(review page, Background: the activation covariance), damping by 1 % of the largest diagonal entry or
of the trace instead of the mean (GPTQ damping), and a block trace that also counts off-diagonal
entries (review page, Method (2): tr(H_G) in the sensitivity score).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle.kronq as kq

import test_oracle_pins as pins


def _damp_max(H, damp=0.01):
    H = np.asarray(H, np.float64)
    lam = damp * float(np.max(np.diag(H)))
    return H + lam * np.eye(H.shape[0]), lam


def _damp_trace(H, damp=0.01):
    H = np.asarray(H, np.float64)
    lam = damp * float(np.trace(H))
    return H + lam * np.eye(H.shape[0]), lam


def _hessian_n1(X):
    X = np.asarray(X, np.float64)
    return X.T @ X / max(X.shape[0] - 1, 1)


def _hessian_sum(X):
    X = np.asarray(X, np.float64)
    return X.T @ X


def _trace_all_entries(HG, form):
    HG = np.asarray(HG, np.float64)
    return float(HG.sum()) if form != "full" else float(np.trace(HG))


MUTATIONS = {
    "damping by the largest diagonal entry": ("damped", _damp_max),
    "damping by the trace": ("damped", _damp_trace),
    "H_X divided by n - 1": ("hessian", _hessian_n1),
    "H_X not divided": ("hessian", _hessian_sum),
    "block trace counting off-diagonal entries": ("trace_form", _trace_all_entries),
}

P18 = [pins.test_p18_hessian_hand_worked, pins.test_p18_damping_hand_worked, pins.test_p18_trace_forms_hand_worked]


def test_pins_pass_on_the_oracle_as_it_stands():
    for pin in P18:
        pin()


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_a_planted_mistake_fails_a_pin(name, monkeypatch):
    attr, wrong = MUTATIONS[name]
    monkeypatch.setattr(kq, attr, wrong)
    failed = []
    for pin in P18:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no hand-worked pin catches: {name}"
