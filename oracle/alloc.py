"""Sublayer mixed-precision allocation driven by tr(H_G) tr(H_X) (oracle).

KronQ review page, Method (2) and Comparison: the joint score tr(H_G) tr(H_X)
drives sublayer-level mixed-precision allocation and yields a "sublayer upgrade
ordering" (Table 6 is not on the pages). The exact rule is not given.

Reading: start every sublayer at the lowest width and repeatedly apply the single
upgrade b -> b + 1 with the largest expected loss reduction per added bit,

    gain_l = sigma_l [c(b_l) - c(b_l + 1)] / n_l,   c(b) = (2^b - 1)^-2,

among the upgrades that still fit the parameter-weighted budget
sum_l n_l b_l <= B sum_l n_l. c(b) is the expected squared rounding error per unit
of squared range for a b-bit grid: zero-mean uniform rounding errors have variance
d^2 / 12 and the range is (2^b - 1) d (Hessian-guided PTQ page, appendix
"Quantization loss decomposition"). Ties go to the earlier sublayer in
(layer, q, k, v, o, gate, up, down) order. Stops when nothing fits.
"""
from __future__ import annotations

import itertools

import numpy as np


def unit_loss(bits: int) -> float:
    return float(2 ** bits - 1) ** -2


def allocate(scores, sizes, budget: float = 3.0, bmin: int = 2, bmax: int = 4) -> np.ndarray:
    scores = np.asarray(scores, dtype=np.float64)
    sizes = np.asarray(sizes, dtype=np.int64)
    b = np.full(len(scores), bmin, dtype=np.int64)
    cap = budget * float(sizes.sum())
    used = float(bmin * sizes.sum())
    while True:
        best, best_gain = -1, -np.inf
        for l in range(len(scores)):
            if b[l] >= bmax or used + sizes[l] > cap:
                continue
            gain = scores[l] * (unit_loss(b[l]) - unit_loss(b[l] + 1)) / sizes[l]
            if gain > best_gain:
                best, best_gain = l, gain
        if best < 0:
            return b
        b[best] += 1
        used += float(sizes[best])


def expected_loss(scores, bits) -> float:
    """sum_l sigma_l c(b_l): the allocation objective (up to the common range factor)."""
    return float(sum(s * unit_loss(int(b)) for s, b in zip(scores, bits)))


def allocate_exact(scores, sizes, budget: float = 3.0, bmin: int = 2, bmax: int = 4) -> np.ndarray:
    """Exhaustive minimum of the objective under the same budget (tiny cases only)."""
    sizes = np.asarray(sizes, dtype=np.int64)
    cap = budget * float(sizes.sum())
    best, best_val = None, np.inf
    for combo in itertools.product(range(bmin, bmax + 1), repeat=len(scores)):
        if float(np.dot(combo, sizes)) > cap:
            continue
        v = expected_loss(scores, combo)
        if v < best_val:
            best, best_val = np.array(combo), v
    return best
