"""Hadamard matrices for the random-sign incoherence rotations (oracle).

The KronQ review page (section "Where this paper sits") traces the input-side
rotation to QuIP/QuIP#, which use Hadamard transforms; the Hessian-guided PTQ
page (Background, "Transformations") lists randomized Hadamard transforms among
the function-preserving orthogonal transforms. Neither page says how a
dimension that is not a power of two is handled.

Reading used here: a true Hadamard matrix of order d = m * 2^k,

    H_d = P_m (x) H_{2^k}                                   (Kronecker product)

where H_{2^k} is Sylvester's matrix in natural order and P_m is a Paley type-I
matrix of order m = q + 1 built over GF(q), q a prime power with q = 3 (mod 4).
m is the smallest order of the form (odd part of d) * 2^a that is 1 or such a
q + 1.

Everything here is integer arithmetic on small tables; the dense matrices are
only built for small d (tests), the structured application is used otherwise.
"""
from __future__ import annotations

from functools import lru_cache

import numpy as np

# Irreducible cubic polynomials used to build GF(p^3): coefficients (c0, c1, c2)
# of x^3 + c2 x^2 + c1 x + c0.
_IRRED3 = {27: (3, (2, 2, 0)),      # x^3 + 2x + 2 over GF(3)
           343: (7, (5, 0, 0))}     # x^3 + 5 over GF(7)


def _is_prime(n: int) -> bool:
    if n < 2:
        return False
    f = 2
    while f * f <= n:
        if n % f == 0:
            return False
        f += 1
    return True


def field_supported(q: int) -> bool:
    return (_is_prime(q) or q in _IRRED3) and q % 4 == 3


def decompose(d: int) -> tuple[int, int]:
    """d -> (m, 2^k) with d = m * 2^k and m the smallest admissible Paley order (or 1)."""
    if d <= 0:
        raise ValueError("dimension must be positive")
    two = d & (-d)
    odd = d // two
    a = 1
    while a <= two:
        m = odd * a
        if m == 1 or field_supported(m - 1):
            return m, d // m
        a *= 2
    raise ValueError(f"no Hadamard order available for d={d}")


def sylvester(n: int) -> np.ndarray:
    """Sylvester's Hadamard matrix of order n = 2^k: H_1 = [1], H_2j = [[H_j, H_j], [H_j, -H_j]]."""
    if n & (n - 1):
        raise ValueError("order must be a power of two")
    H = np.ones((1, 1), dtype=np.int64)
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def _gf_elements(q: int):
    """Return (p, e, mul) with elements indexed by base-p digits a0 + p a1 + p^2 a2."""
    if _is_prime(q):
        return q, 1, None
    p, (c0, c1, c2) = _IRRED3[q]

    def digits(k):
        return [k % p, (k // p) % p, k // (p * p)]

    def mul(a, b):
        x, y = digits(a), digits(b)
        prod = [0] * 5
        for i in range(3):
            for j in range(3):
                prod[i + j] = (prod[i + j] + x[i] * y[j]) % p
        # reduce x^4 and x^3 with x^3 = -(c2 x^2 + c1 x + c0)
        for deg in (4, 3):
            c = prod[deg]
            if c:
                prod[deg] = 0
                prod[deg - 1] = (prod[deg - 1] - c * c2) % p
                prod[deg - 2] = (prod[deg - 2] - c * c1) % p
                prod[deg - 3] = (prod[deg - 3] - c * c0) % p
        return prod[0] + p * prod[1] + p * p * prod[2]

    return p, 3, mul


def gf_sub(q: int, a: int, b: int) -> int:
    p, e, _ = _gf_elements(q)
    out, place = 0, 1
    for _ in range(e):
        out += ((a % p - b % p) % p) * place
        a //= p
        b //= p
        place *= p
    return out


def quadratic_character(q: int) -> np.ndarray:
    """chi over GF(q) by element index: 0 at 0, +1 on nonzero squares, -1 otherwise."""
    p, e, mul = _gf_elements(q)
    chi = -np.ones(q, dtype=np.int64)
    chi[0] = 0
    for y in range(1, q):
        sq = (y * y) % q if mul is None else mul(y, y)
        chi[sq] = 1
    return chi


@lru_cache(maxsize=None)
def paley(m: int) -> np.ndarray:
    """Paley type-I Hadamard matrix of order m = q + 1: P = I + [[0, 1^T], [-1, Q]], Q_ab = chi(a - b)."""
    q = m - 1
    if not field_supported(q):
        raise ValueError(f"no Paley construction for order {m}")
    chi = quadratic_character(q)
    Q = np.empty((q, q), dtype=np.int64)
    for a in range(q):
        for b in range(q):
            Q[a, b] = chi[gf_sub(q, a, b)]
    S = np.zeros((m, m), dtype=np.int64)
    S[0, 1:] = 1
    S[1:, 0] = -1
    S[1:, 1:] = Q
    return np.eye(m, dtype=np.int64) + S


def hadamard(d: int) -> np.ndarray:
    """Dense H_d = P_m (x) H_{2^k} (small d only)."""
    m, p2 = decompose(d)
    Pm = np.ones((1, 1), dtype=np.int64) if m == 1 else paley(m)
    return np.kron(Pm, sylvester(p2))


def _fwht_last(x: np.ndarray) -> np.ndarray:
    """y = H_{2^k} x along the last axis, following the Sylvester recursion directly."""
    n = x.shape[-1]
    if n == 1:
        return x.copy()
    top = _fwht_last(x[..., : n // 2])
    bot = _fwht_last(x[..., n // 2:])
    return np.concatenate([top + bot, top - bot], axis=-1)


def apply(x: np.ndarray, axis: int = -1, transpose: bool = False) -> np.ndarray:
    """y = H_d x (or H_d^T x) along ``axis`` of a float64 array, unnormalised.

    With index j = a * 2^k + b, (P_m (x) H_{2^k})[(a,b),(a',b')] = P[a,a'] H[b,b']:
    every contiguous 2^k chunk is transformed by H_{2^k}, then chunks are mixed by P_m.
    """
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
    d = x.shape[-1]
    m, p2 = decompose(d)
    y = _fwht_last(x.reshape(x.shape[:-1] + (m, p2)))
    if m > 1:
        P = paley(m).astype(np.float64)
        if transpose:
            P = P.T
        y = np.matmul(P, y)
    return np.moveaxis(y.reshape(x.shape), -1, axis)
