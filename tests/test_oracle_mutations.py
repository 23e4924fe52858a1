"""The oracle's pins catch plausible mistakes anywhere along the path.

Each case plants one mistake in the oracle (on the CPU, for the duration of the test only) and checks
that at least one of the pins named for it then fails. The mistakes: H_X = X^T X / n divided by n - 1
or not at all (review page, Background); damping by 1 % of the largest diagonal entry or of the trace
instead of the mean (GPTQ damping); the rotation without its 1/sqrt(d) or with the Hadamard matrix
transposed (review page, "Where this paper sits": random Hadamard rotations); S and S^-1 exchanged
(review page, Method (1): the H_G^{1/2} transform); the factor of H instead of H^-1, or its lower
instead of its upper form (GPTQ's Cholesky form of the inverse Hessian); a grid step over 2^b levels
instead of 2^b - 1, and rounding halves away from zero instead of to even (Hessian-guided PTQ page,
Background: grid step and shift); the error propagated with the wrong sign, in the per-column and in
the blocked sweep (review page, Prior limitations: the column-wise OBS update); codes packed from the
most significant bit; the score as a sum instead of a product and a block trace that counts
off-diagonal entries (review page, Method (2)); the bit upgrades taken by the smallest gain.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle.alloc as al
import oracle.hadamard as hd
import oracle.kronq as kq

import test_oracle_pins as pins

_ORIG = {
    "inverse_upper_factor": kq.inverse_upper_factor,
    "sweep_plain": kq.sweep_plain,
    "sweep_blocked": kq.sweep_blocked,
    "_rot": kq._rot,
    "hg_sqrt": kq.hg_sqrt,
    "pack": kq.pack,
    "apply": hd.apply,
}


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


def _score_sum(HX, HG, form):
    return kq.trace_form(HG, form) + float(np.trace(np.asarray(HX, np.float64)))


def _factor_of_H(H):
    return np.linalg.cholesky(np.asarray(H, np.float64)).T


def _factor_lower(H):
    return _ORIG["inverse_upper_factor"](H).T


def _grid_2b(v, bits):
    mu = v.min(axis=-1)
    return mu, (v.max(axis=-1) - mu) / 2 ** bits


def _round_half_away(w, mu, s, bits):
    L = 2 ** bits - 1
    pos = s > 0
    u = np.where(pos, (w - mu) / np.where(pos, s, 1.0), 0.0)
    q = np.where(pos, np.clip(np.floor(u + 0.5), 0, L), 0.0)
    delta = np.where(pos, np.abs(u - (np.floor(u) + 0.5)), np.inf)
    return q.astype(np.int64), mu + s * q, delta


def _flip_offdiag(R):
    # the sweeps subtract e R[j, j+1:]; negating R off its diagonal adds it instead
    R = np.asarray(R, np.float64)
    return 2.0 * np.diag(np.diag(R)) - R


def _sweep_plain_flipped(W2, R, *a, **k):
    return _ORIG["sweep_plain"](W2, _flip_offdiag(R), *a, **k)


def _sweep_blocked_flipped(W2, R, *a, **k):
    return _ORIG["sweep_blocked"](W2, _flip_offdiag(R), *a, **k)


def _rot_unnormalised(x, sign, axis):
    return _ORIG["_rot"](x, sign, axis) * np.sqrt(np.asarray(x).shape[axis])


def _roots_swapped(HG, form):
    S, Si = _ORIG["hg_sqrt"](HG, form)
    return Si, S


def _pack_msb_first(codes, bits):
    c = np.asarray(codes, np.int64)
    rev = np.zeros_like(c)
    for k in range(bits):
        rev |= ((c >> k) & 1) << (bits - 1 - k)
    return _ORIG["pack"](rev, bits)


def _apply_transposed(x, axis=-1, transpose=False):
    return _ORIG["apply"](x, axis=axis, transpose=not transpose)


def _allocate_smallest_gain(scores, sizes, budget=3.0, bmin=2, bmax=4):
    scores = np.asarray(scores, np.float64)
    sizes = np.asarray(sizes, np.int64)
    b = np.full(len(scores), bmin, dtype=np.int64)
    cap, used = budget * float(sizes.sum()), float(bmin * sizes.sum())
    while True:
        best, best_gain = -1, np.inf
        for l in range(len(scores)):
            if b[l] >= bmax or used + sizes[l] > cap:
                continue
            gain = scores[l] * (al.unit_loss(b[l]) - al.unit_loss(b[l] + 1)) / sizes[l]
            if gain < best_gain:
                best, best_gain = l, gain
        if best < 0:
            return b
        b[best] += 1
        used += float(sizes[best])


P18 = [pins.test_p18_hessian_hand_worked, pins.test_p18_damping_hand_worked, pins.test_p18_trace_forms_hand_worked]
P5 = [lambda: pins.test_p5_cholesky_sweep_equals_naive_obs(3, 0), pins.test_p5_upper_factor_closed_form_2x2]

# mistake -> (module, attribute, wrong version, pins expected to catch it)
MUTATIONS = {
    "damping by the largest diagonal entry": (kq, "damped", _damp_max, P18),
    "damping by the trace": (kq, "damped", _damp_trace, P18),
    "H_X divided by n - 1": (kq, "hessian", _hessian_n1, P18),
    "H_X not divided": (kq, "hessian", _hessian_sum, P18),
    "block trace counting off-diagonal entries": (kq, "trace_form", _trace_all_entries, P18),
    "score as a sum": (kq, "sensitivity", _score_sum, [pins.test_p10_score_is_expected_loss_coefficient]),
    "factor of H instead of H^-1": (kq, "inverse_upper_factor", _factor_of_H, P5),
    "lower factor instead of upper": (kq, "inverse_upper_factor", _factor_lower, P5),
    "grid step over 2^b levels": (kq, "grid_params", _grid_2b, [pins.test_grid_worked_example]),
    "rounding halves away from zero": (kq, "quantize", _round_half_away, [pins.test_grid_worked_example]),
    "per-column sweep adds the error": (kq, "sweep_plain", _sweep_plain_flipped, P5),
    "blocked sweep adds the error": (kq, "sweep_blocked", _sweep_blocked_flipped,
                                     [pins.test_p6_row_loss_is_damped_quadratic_form] + P5),
    "rotation without 1/sqrt(d)": (kq, "_rot", _rot_unnormalised,
                                   [pins.test_p4_square_root_and_loss_in_both_coordinates]),
    "S and S^-1 exchanged": (kq, "hg_sqrt", _roots_swapped, [pins.test_p4_square_root_and_loss_in_both_coordinates]),
    "Hadamard matrix transposed": (hd, "apply", _apply_transposed,
                                   [lambda: pins.test_p2_hadamard_orthogonality_and_fast_apply(12)]),
    "codes packed from the most significant bit": (kq, "pack", _pack_msb_first,
                                                   [pins.test_pack_matches_big_integer_bitstream]),
    "bit upgrades by the smallest gain": (al, "allocate", _allocate_smallest_gain, [pins.test_p11_allocation]),
}


def test_named_pins_pass_on_the_oracle_as_it_stands():
    for _, _, _, named in MUTATIONS.values():
        for pin in named:
            pin()


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_a_planted_mistake_fails_a_pin(name, monkeypatch):
    mod, attr, wrong, named = MUTATIONS[name]
    monkeypatch.setattr(mod, attr, wrong)
    failed = 0
    for pin in named:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed, f"no pin catches: {name}"
