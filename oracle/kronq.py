"""Float64 oracle of the per-layer KronQ solver.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests, the
smoke check and the CPU-baseline leg of the benchmark, never by the GPU library.

Notation. W is o x i (row r = output channel, y = W x), X is n x i, H_X = X^T X / n,
H_G is o x o symmetric positive definite, and the layer loss under the
Kronecker-factored Hessian H ~ H_X (x) H_G is

    L(W^) = tr(H_G dW H_X dW^T),   dW = W^ - W

(KronQ review page, Background: "the full weight Hessian factorizes as H ~ H_X (x)
H_G"; GPTQ-style methods take H_G = I). With column-stacking vec, vec(dW)^T (H_X (x)
H_G) vec(dW) equals that trace.

Pipeline (KronQ review page, Method and Key idea; spec reading):
  1. H_X from the calibration activations.
  2. Input side: W' = W U, H_X' = U^T H_X U with U = D_s H_i^T / sqrt(i).
  3. Output side: W'' = V S W' with S = H_G^{1/2} (principal root), V = H_o D_t / sqrt(o).
     Then S^{-T} H_G S^{-1} = I, so L = tr(dW'' H_X' dW''^T): a plain GPTQ loss
     ("H_G cancels out of the quantization update", review page, Method).
  4. Damped H = H_X' + lambda I, lambda = 0.01 mean diag; R upper with H^{-1} = R^T R.
  5. Column sweep on W'' with R (GPTQ; the review page's Prior limitations / Goal:
     the solver itself is unchanged).
  6. Sensitivity tr(H_G) tr(H_X) (review page, Method (2)).
"""
from __future__ import annotations

import numpy as np

from . import hadamard

# ============================================================================= step 1: H_X


def hessian(X: np.ndarray) -> np.ndarray:
    """H_X = X^T X / n in float64 from the exact input values (review page, Background:
    the input activation covariance used as the layer-Hessian proxy)."""
    X = np.asarray(X, dtype=np.float64)
    return X.T @ X / X.shape[0]


# ============================================================================= step 2: input rotation


def _rot(x: np.ndarray, sign: np.ndarray, axis: int) -> np.ndarray:
    """x -> H_d (sign * x) / sqrt(d) along ``axis``."""
    d = x.shape[axis]
    shape = [1] * x.ndim
    shape[axis] = d
    return hadamard.apply(x * np.asarray(sign, dtype=np.float64).reshape(shape), axis=axis) / np.sqrt(d)


def _unrot(x: np.ndarray, sign: np.ndarray, axis: int) -> np.ndarray:
    """Inverse of ``_rot``: x -> sign * (H_d^T x) / sqrt(d)."""
    d = x.shape[axis]
    shape = [1] * x.ndim
    shape[axis] = d
    return hadamard.apply(x, axis=axis, transpose=True) / np.sqrt(d) * np.asarray(sign, np.float64).reshape(shape)


def rotation_matrix(sign: np.ndarray) -> np.ndarray:
    """U = D_s H_d^T / sqrt(d) as a dense matrix (small d only)."""
    d = len(sign)
    return np.diag(np.asarray(sign, np.float64)) @ hadamard.hadamard(d).T.astype(np.float64) / np.sqrt(d)


def rotate_in_weights(W: np.ndarray, s: np.ndarray) -> np.ndarray:
    """W' = W U: every row w -> H_i (s * w) / sqrt(i) (review page, "Where this paper sits":
    the QuIP/QuIP# input-side random Hadamard incoherence rotation)."""
    return _rot(np.asarray(W, np.float64), s, axis=1)


def rotate_in_hessian(HX: np.ndarray, s: np.ndarray) -> np.ndarray:
    """H_X' = U^T H_X U (curvature transforms by congruence; Hessian-guided PTQ page,
    appendix "Range clipping for weights derivation": G_{W_T} = T^T G_W)."""
    A = _rot(np.asarray(HX, np.float64), s, axis=1)    # H_X U   (rows)
    return _rot(A, s, axis=0)                          # U^T (.) (columns)


# ============================================================================= step 3: output transform


def hg_sqrt(HG: np.ndarray, form: str) -> tuple[np.ndarray, np.ndarray]:
    """S = H_G^{1/2} (principal, symmetric positive definite) and S^{-1}, in the storage form
    of H_G: diag -> (o,), block -> (nb, b, b), full -> (o, o).

    The pages only write H_G^{1/2}; the principal root is its literal meaning."""
    HG = np.asarray(HG, np.float64)
    if form == "diag":
        if np.any(HG <= 0):
            raise np.linalg.LinAlgError("H_G not positive definite")
        return np.sqrt(HG), 1.0 / np.sqrt(HG)

    def one(A):
        lam, Q = np.linalg.eigh(0.5 * (A + A.T))
        if lam[0] <= 0:
            raise np.linalg.LinAlgError("H_G not positive definite")
        return (Q * np.sqrt(lam)) @ Q.T, (Q / np.sqrt(lam)) @ Q.T

    if form == "block":
        S = np.empty_like(HG)
        Si = np.empty_like(HG)
        for k in range(HG.shape[0]):
            S[k], Si[k] = one(HG[k])
        return S, Si
    if form == "full":
        return one(HG)
    raise ValueError(form)


def form_matmul(S: np.ndarray, form: str, M: np.ndarray) -> np.ndarray:
    """S @ M for S in diag / block / full storage form; M has o rows."""
    M = np.asarray(M, np.float64)
    if form == "diag":
        return S[:, None] * M
    if form == "block":
        nb, b, _ = S.shape
        return np.einsum("kab,kbc->kac", S, M.reshape(nb, b, -1)).reshape(M.shape)
    return S @ M


def form_dense(S: np.ndarray, form: str) -> np.ndarray:
    if form == "diag":
        return np.diag(S)
    if form == "block":
        nb, b, _ = S.shape
        out = np.zeros((nb * b, nb * b))
        for k in range(nb):
            out[k * b:(k + 1) * b, k * b:(k + 1) * b] = S[k]
        return out
    return np.asarray(S)


def rotate_out(W1: np.ndarray, S: np.ndarray, form: str, t: np.ndarray) -> np.ndarray:
    """W'' = V S W' with V = H_o D_t / sqrt(o), applied along the output axis (KronQ abstract:
    the input-side rotation is extended to the output dimension using the gradient covariance)."""
    return _rot(form_matmul(S, form, W1), t, axis=0)


# ============================================================================= step 4: damping and factor


def damped(HX2: np.ndarray, damp: float = 0.01) -> tuple[np.ndarray, float]:
    """H = H_X'' + lambda I with lambda = damp * mean(diag H_X'') (GPTQ damping)."""
    HX2 = np.asarray(HX2, np.float64)
    lam = damp * float(np.mean(np.diag(HX2)))
    return HX2 + lam * np.eye(HX2.shape[0]), lam


def inverse_upper_factor(H: np.ndarray) -> np.ndarray:
    """R: the upper-triangular matrix with positive diagonal such that H^{-1} = R^T R
    (GPTQ's Cholesky form of the inverse Hessian). Definition written out."""
    Hinv = np.linalg.inv(np.asarray(H, np.float64))
    Hinv = 0.5 * (Hinv + Hinv.T)
    return np.linalg.cholesky(Hinv).T


# ============================================================================= step 5: grid and sweep


def grid_params(v: np.ndarray, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """Asymmetric min-max grid over the last axis: shift mu = min v, step s = (max v - min v) / (2^b - 1)
    (Hessian-guided PTQ page, Background: a grid step s and a shift mu; asymmetric shifted grid)."""
    mu = v.min(axis=-1)
    return mu, (v.max(axis=-1) - mu) / (2 ** bits - 1)


def quantize(w: np.ndarray, mu: np.ndarray, s: np.ndarray, bits: int):
    """Round to the grid: q = clamp(rne((w - mu) / s), 0, 2^b - 1), w^ = mu + s q; s = 0 gives q = 0.
    Also returns the tie distance |u - (floor(u) + 1/2)| in grid steps."""
    L = 2 ** bits - 1
    pos = s > 0
    u = np.where(pos, (w - mu) / np.where(pos, s, 1.0), 0.0)
    q = np.clip(np.rint(u), 0, L)
    q = np.where(pos, q, 0.0)
    delta = np.where(pos, np.abs(u - (np.floor(u) + 0.5)), np.inf)
    return q.astype(np.int64), mu + s * q, delta


def search_alphas(M: int) -> np.ndarray:
    """The candidate range factors: M values spread evenly over [1/2, 1] (1 alone for M = 1)."""
    return 0.5 + 0.5 * np.arange(M) / (M - 1) if M > 1 else np.ones(1)


def grid_search(v: np.ndarray, d: np.ndarray, bits: int, M: int, near_scale: np.ndarray | None = None):
    """Hessian-aware choice of the grid of each row of v (H_Z-PTQ page, Weight scales and rounding:
    a grid search over a few candidate scales for the one with the smallest curvature-weighted
    rounding error; its experimental settings: 500 candidates spread evenly over [max|w|, 2 max|w|],
    i.e. one half to all of the full range). Asymmetric reading for the shifted grid here: the
    [min, max] range is shrunk about its midpoint by alpha in [1/2, 1]; the weight of column c is
    d_c, the curvature the sweep charges an error in column c with (1 / R_cc^2). alpha = 1 is the
    min-max grid, so the chosen grid never has a larger weighted rounding error.

    Returns mu, s, the chosen candidate index and every candidate's objective (rows x M). With
    ``near_scale`` the candidate whose step is nearest to it is taken instead of the argmin (replay
    of another implementation's choice; the caller checks its objective)."""
    L = 2 ** bits - 1
    mn, mx = v.min(axis=-1), v.max(axis=-1)
    c, h = (mn + mx) / 2, (mx - mn) / 2
    alphas = search_alphas(M)
    obj = np.empty((v.shape[0], M))
    for m, a in enumerate(alphas):
        mu_a, s_a = c - a * h, 2 * a * h / L
        _, deq, _ = quantize(v, mu_a[:, None], s_a[:, None], bits)
        obj[:, m] = ((v - deq) ** 2 * d[None, :]).sum(axis=-1)
    idx = obj.argmin(axis=-1)
    if near_scale is not None:
        steps = 2 * alphas[None, :] * h[:, None] / L
        idx = np.abs(steps - np.asarray(near_scale, np.float64)[:, None]).argmin(axis=-1)
    a = alphas[idx]
    return c - a * h, 2 * a * h / L, idx, obj


def sweep_plain(W2: np.ndarray, R: np.ndarray, bits: int, group: int = 0,
                force_mask: np.ndarray | None = None, force_codes: np.ndarray | None = None,
                stop: int | None = None) -> dict:
    """GPTQ column sweep, per-column definition (KronQ review page, Prior limitations: GPTQ
    solves the column-wise OBS update using H_X; "Where this paper sits": GPTQ recast the OBS
    update column-wise). For j = 0..i-1:

        at a group start set (mu, s) from the current W[:, j:j+g]  (per-row grids: once, before)
        q_j = Q(W[:, j]);  e = (W[:, j] - w^_j) / R_jj
        W[:, j+1:] -= e R[j, j+1:];  W[:, j] = w^_j;  row_loss += e^2

    ``force_mask``/``force_codes`` (o x i) override the rounding decision at given positions
    (used to replay a row after a near-tie flip). ``stop`` ends the sweep after that many columns
    and returns the partially updated matrix (columns >= stop still continuous)."""
    W = np.array(W2, dtype=np.float64)
    o, i = W.shape
    ng = i // group if group else 1
    codes = np.zeros((o, i), dtype=np.int64)
    delta = np.zeros((o, i))
    mu_all = np.zeros((o, ng))
    sc_all = np.zeros((o, ng))
    loss = np.zeros(o)
    if not group:
        mu, s = grid_params(W, bits)
        mu_all[:, 0], sc_all[:, 0] = mu, s
    for j in range(i if stop is None else stop):
        if group and j % group == 0:
            mu, s = grid_params(W[:, j:j + group], bits)
            mu_all[:, j // group], sc_all[:, j // group] = mu, s
        q, deq, dl = quantize(W[:, j], mu, s, bits)
        if force_mask is not None and force_mask[:, j].any():
            f = force_mask[:, j]
            q = q.copy()
            q[f] = force_codes[f, j]
            deq = mu + s * q
        e = (W[:, j] - deq) / R[j, j]
        W[:, j + 1:] -= np.outer(e, R[j, j + 1:])
        W[:, j] = deq
        codes[:, j], delta[:, j] = q, dl
        loss += e * e
    return {"codes": codes, "mu": mu_all, "scale": sc_all, "Q": W, "row_loss": loss, "delta": delta}


def sweep_blocked(W2: np.ndarray, R: np.ndarray, bits: int, group: int = 0, block: int = 128,
                  force_mask: np.ndarray | None = None, force_codes: np.ndarray | None = None,
                  search: int = 0, near_scale: np.ndarray | None = None) -> dict:
    """Same sweep with GPTQ's lazy batch updates over ``block`` columns: in-block steps update only
    the block's own columns, and after the block W[:, b1:] -= E R[b0:b1, b1:] (spec:
    "lazy trailing updates W[:, j+B:] -= E Hinv[B, j+B:]"). Exactly equal to ``sweep_plain`` in exact
    arithmetic when group divides block or block divides group.

    ``search`` > 0 chooses every grid by ``grid_search`` over that many candidates with the column
    weights 1 / R_cc^2 instead of min-max; ``near_scale`` (o x groups) replays given steps there."""
    W = np.array(W2, dtype=np.float64)
    o, i = W.shape
    if group and (block % group) and (group % block):
        raise ValueError("group and block must divide one another")
    ng = i // group if group else 1
    codes = np.zeros((o, i), dtype=np.int64)
    delta = np.zeros((o, i))
    mu_all = np.zeros((o, ng))
    sc_all = np.zeros((o, ng))
    loss = np.zeros(o)
    dw = 1.0 / np.diag(np.asarray(R, np.float64)) ** 2
    chosen = np.zeros((o, ng), dtype=np.int64)
    objs = np.zeros((o, ng, max(search, 1)))

    def pick(v, dcol, g):
        if not search:
            return grid_params(v, bits)
        ns = None if near_scale is None else near_scale[:, g]
        m, st, idx, obj = grid_search(v, dcol, bits, search, ns)
        chosen[:, g], objs[:, g] = idx, obj
        return m, st
    if not group:
        mu, s = pick(W, dw, 0)
        mu_all[:, 0], sc_all[:, 0] = mu, s
    for b0 in range(0, i, block):
        b1 = min(b0 + block, i)
        E = np.zeros((o, b1 - b0))
        for j in range(b0, b1):
            if group and j % group == 0:
                mu, s = pick(W[:, j:j + group], dw[j:j + group], j // group)
                mu_all[:, j // group], sc_all[:, j // group] = mu, s
            q, deq, dl = quantize(W[:, j], mu, s, bits)
            if force_mask is not None and force_mask[:, j].any():
                f = force_mask[:, j]
                q = q.copy()
                q[f] = force_codes[f, j]
                deq = mu + s * q
            e = (W[:, j] - deq) / R[j, j]
            W[:, j + 1:b1] -= np.outer(e, R[j, j + 1:b1])
            W[:, j] = deq
            E[:, j - b0] = e
            codes[:, j], delta[:, j] = q, dl
            loss += e * e
        if b1 < i:
            W[:, b1:] -= E @ R[b0:b1, b1:]
    out = {"codes": codes, "mu": mu_all, "scale": sc_all, "Q": W, "row_loss": loss, "delta": delta}
    if search:
        out["chosen"], out["objectives"] = chosen, objs
    return out


def sweep_obs_naive(W2: np.ndarray, H: np.ndarray, bits: int, group: int = 0) -> dict:
    """Optimal Brain Surgeon sweep with an explicitly maintained inverse (the principle GPTQ
    recasts column-wise; review page, "Where this paper sits"). For each column j in order:
    quantize, update the remaining free weights w_F -= (w_j - w^_j) / Hinv_jj * Hinv_{j,F}, then
    remove j: Hinv <- Hinv - Hinv_{:,j} Hinv_{j,:} / Hinv_jj. Slow; small cases only."""
    W = np.array(W2, dtype=np.float64)
    o, i = W.shape
    Hinv = np.linalg.inv(np.asarray(H, np.float64))
    codes = np.zeros((o, i), dtype=np.int64)
    loss = np.zeros(o)
    if not group:
        mu, s = grid_params(W, bits)
    for j in range(i):
        if group and j % group == 0:
            mu, s = grid_params(W[:, j:j + group], bits)
        q, deq, _ = quantize(W[:, j], mu, s, bits)
        err = W[:, j] - deq
        d = Hinv[j, j]
        W[:, j + 1:] -= np.outer(err / d, Hinv[j, j + 1:])
        W[:, j] = deq
        loss += err * err / d
        Hinv = Hinv - np.outer(Hinv[:, j], Hinv[j, :]) / d
        codes[:, j] = q
    return {"codes": codes, "Q": W, "row_loss": loss}


# ============================================================================= packing


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """Row-major b-bit codes -> little-endian uint32 words, LSB-first bit stream per row,
    each row starting on a word boundary (requires i * b to be a multiple of 32)."""
    o, i = codes.shape
    if (i * bits) % 32:
        raise ValueError("i * bits must be a multiple of 32")
    words = np.zeros((o, i * bits // 32), dtype=np.uint64)
    for j in range(i):
        for t in range(bits):
            pos = j * bits + t
            bit = (codes[:, j].astype(np.uint64) >> np.uint64(t)) & np.uint64(1)
            words[:, pos // 32] |= bit << np.uint64(pos % 32)
    return words.astype(np.uint32)


def unpack(words: np.ndarray, bits: int, i: int) -> np.ndarray:
    w = words.astype(np.uint64)
    out = np.zeros((w.shape[0], i), dtype=np.int64)
    for j in range(i):
        for t in range(bits):
            pos = j * bits + t
            out[:, j] |= (((w[:, pos // 32] >> np.uint64(pos % 32)) & np.uint64(1)) << np.uint64(t)).astype(np.int64)
    return out


def dequantize(codes: np.ndarray, mu: np.ndarray, scale: np.ndarray, group: int) -> np.ndarray:
    """w^ = mu + s q with the group (or per-row) parameters."""
    o, i = codes.shape
    g = group if group else i
    return np.repeat(mu, g, axis=1)[:, :i] + np.repeat(scale, g, axis=1)[:, :i] * codes


# ============================================================================= verification


def unrotate(Q2: np.ndarray, s: np.ndarray, t: np.ndarray, Sinv: np.ndarray, form: str) -> np.ndarray:
    """W^ = S^{-1} V^T Q'' U^T: the dequantized weights in the original coordinates."""
    A = _unrot(np.asarray(Q2, np.float64), t, axis=0)      # V^T Q''
    A = form_matmul(Sinv, form, A)                          # S^{-1} (.)
    return _unrot(A, s, axis=1)                             # (.) U^T: row a -> s * (H_i^T a) / sqrt(i)


# ============================================================================= H_G preparation


def hg_forms(H: np.ndarray, form: str, blk: int = 128) -> np.ndarray:
    """Storage form of an o x o covariance: the matrix, its blk x blk diagonal blocks, or its
    diagonal (KronQ review page, Sparks: blockwise approximations of H_G)."""
    H = np.asarray(H)
    o = H.shape[0]
    if form == "full":
        return H.copy()
    if form == "block":
        return np.stack([H[b:b + blk, b:b + blk] for b in range(0, o, blk)])
    return np.diag(H).copy()


def _sym_fn(A: np.ndarray, f) -> np.ndarray:
    w, V = np.linalg.eigh((A + A.T) / 2)
    return (V * f(w)) @ V.T


def hg_lowrank(G: np.ndarray, k: int, q: int, omega: np.ndarray) -> dict:
    """Low-rank-plus-isotropic approximation of H = G^T G / n (KronQ review page, Sparks: low-rank
    approximations of H_G; the form below is this build's reading). The range of H^{q+1} Omega is
    found step by step (re-orthonormalised after every product with H, which leaves the range
    unchanged); with Q its orthonormal basis, B = Q^T H Q and sigma = (tr H - tr B) / (o - k),
    H^ = Q B Q^T + sigma (I - Q Q^T). S and S^{-1} are the principal square root of H^ and its
    inverse, taken from H^'s eigendecomposition."""
    G = np.asarray(G, np.float64)
    n, o = G.shape
    H = G.T @ G / n
    Q, _ = np.linalg.qr(H @ np.asarray(omega, np.float64))
    for _ in range(q):
        Q, _ = np.linalg.qr(H @ Q)
    B = Q.T @ H @ Q
    sigma = (np.trace(H) - np.trace(B)) / (o - k)
    Hhat = Q @ B @ Q.T + sigma * (np.eye(o) - Q @ Q.T)
    out = {"H": H, "Hhat": Hhat, "sigma": float(sigma), "trH": float(np.trace(H)), "Q": Q, "B": B}
    if sigma > 0:
        out["S"] = _sym_fn(Hhat, np.sqrt)
        out["Sinv"] = _sym_fn(Hhat, lambda w: 1.0 / np.sqrt(w))
    return out


def matvec_quantized(words: np.ndarray, mu: np.ndarray, scale: np.ndarray, bits: int, group: int, s: np.ndarray,
                     t: np.ndarray, Sinv: np.ndarray, form: str, X: np.ndarray) -> np.ndarray:
    """Inference-side product Y = X W^^T for token rows X (n x i), from the packed codes.

    KronQ review page, Limitations (3): at inference the stored Q'' is used through the
    reverted transforms, W^ = S^{-1} V^T Q'' U^T. Written as the definition: decode the codes,
    dequantize, revert the rotations and H_G^{1/2}, then multiply."""
    X = np.asarray(X, np.float64)
    Q2 = dequantize(unpack(words, bits, X.shape[1]), np.asarray(mu, np.float64), np.asarray(scale, np.float64), group)
    What = unrotate(Q2, s, t, Sinv, form)
    return X @ What.T


def kfac_loss(W: np.ndarray, What: np.ndarray, HX: np.ndarray, HG: np.ndarray, form: str) -> float:
    """tr(H_G dW H_X dW^T) with the undamped H_X."""
    dW = np.asarray(What, np.float64) - np.asarray(W, np.float64)
    A = dW @ np.asarray(HX, np.float64)                     # o x i
    B = form_matmul(np.asarray(HG, np.float64), form, dW)   # H_G dW
    return float(np.sum(B * A))


def rotated_loss(W2: np.ndarray, Q2: np.ndarray, HX2: np.ndarray) -> np.ndarray:
    """Per-row dw''_r H dw''_r^T (sum over rows = tr(dW'' H dW''^T))."""
    dW = np.asarray(Q2, np.float64) - np.asarray(W2, np.float64)
    return np.einsum("ri,ri->r", dW @ np.asarray(HX2, np.float64), dW)


# ============================================================================= step 6: sensitivity


def trace_form(HG: np.ndarray, form: str) -> float:
    HG = np.asarray(HG, np.float64)
    if form == "diag":
        return float(HG.sum())
    if form == "block":
        return float(np.einsum("kaa->", HG))
    return float(np.trace(HG))


def sensitivity(HX: np.ndarray, HG: np.ndarray, form: str) -> float:
    """tr(H_G) tr(H_X), both undamped (review page, Method (2): the joint sensitivity metric)."""
    return trace_form(HG, form) * float(np.trace(np.asarray(HX, np.float64)))


# ============================================================================= whole layer


def drift_target(W: np.ndarray, X: np.ndarray, Xt: np.ndarray, damp: float = 0.01) -> dict:
    """Target of the input-drift correction (KronQ review page, Prior limitations: GPTAQ corrects for
    the drift of the input caused by quantizing earlier layers; the formula is not on the pages, so
    this follows the reading that the layer should reproduce W X^T from the drifted inputs X~):
    || W^ X~^T - W X^T ||^2 + n lambda ||W^||^2 is minimised by W* = W C (H~ + lambda I)^{-1},
    C = X^T X~ / n, H~ = X~^T X~ / n, lambda = damp mean diag H~; the sweep then runs on (W*, H~)."""
    X = np.asarray(X, np.float64)
    Xt = np.asarray(Xt, np.float64)
    n = X.shape[0]
    C = X.T @ Xt / n
    Ht = Xt.T @ Xt / n
    H, lam = damped(Ht, damp)
    return {"W": np.asarray(W, np.float64) @ C @ np.linalg.inv(H), "C": C, "H": Ht, "lam": lam}


def block_trace_order(H: np.ndarray, width: int = 128) -> np.ndarray:
    """Blocks of `width` columns in descending order of the trace of their diagonal part of H (ties:
    lower index first). H_Z-PTQ page, Weight scales and rounding: the blocks with larger curvature
    traces are quantized first (GPTQ's act-order at block granularity)."""
    d = np.diag(np.asarray(H, np.float64))
    tr = d.reshape(-1, width).sum(axis=1)
    return np.lexsort((np.arange(tr.size), -tr))


def block_perm_index(order: np.ndarray, width: int) -> np.ndarray:
    """Column index of the permuted matrix: position k * width + c holds column order[k] * width + c."""
    return (np.asarray(order)[:, None] * width + np.arange(width)[None, :]).ravel()


def sweep_trace_order(W2: np.ndarray, H: np.ndarray, bits: int, group: int, block: int = 128, search: int = 0,
                      order: np.ndarray | None = None) -> dict:
    """The sweep with blocks taken in trace order: permute the columns of W'' and both axes of the
    damped H by blocks, factor and sweep there, and put the results back in the natural order (the
    codes and grids of a block move with it, since groups and packed words stay inside blocks)."""
    o, i = W2.shape
    if order is None:
        order = block_trace_order(H, block)
    p = block_perm_index(order, block)
    Hp = np.asarray(H, np.float64)[np.ix_(p, p)]
    R = inverse_upper_factor(Hp)
    sw = sweep_blocked(np.asarray(W2, np.float64)[:, p], R, bits, group, block, search=search)
    inv = np.argsort(p)
    out = dict(sw)
    out["Q"] = sw["Q"][:, inv]
    out["codes"] = sw["codes"][:, inv]
    out["delta"] = sw["delta"][:, inv]
    if group:
        gp = block_perm_index(order, block // group) if block >= group else None
        ginv = np.argsort(gp)
        out["mu"], out["scale"] = sw["mu"][:, ginv], sw["scale"][:, ginv]
    out["order"], out["R_perm"] = np.asarray(order), R
    return out


def quantize_layer(X, W, HG, form: str, s, t, bits: int, group: int, block: int = 128,
                   damp: float = 0.01, rotate_in: bool = True, rotate_out_on: bool = True,
                   mode: str = "blocked", verify: bool = True, search: int = 0, order: str = "natural",
                   Xt=None) -> dict:
    """All steps of the per-layer solver on float64 copies of the inputs. ``search``: candidates of
    the Hessian-aware grid search (0: min-max); ``order``: "natural" or "trace" (blocks in descending
    trace of the damped, rotated H_X); ``Xt``: drifted inputs (the sweep then runs on the drift
    target W* with H~ = X~^T X~ / n)."""
    W = np.asarray(W, np.float64)
    if Xt is not None:
        dr = drift_target(W, X, Xt, damp)
        HX, W = dr["H"], dr["W"]
    else:
        HX = hessian(X)
    o, i = W.shape
    if rotate_in:
        W1, HX2 = rotate_in_weights(W, s), rotate_in_hessian(HX, s)
    else:
        W1, HX2 = W.copy(), HX.copy()
    S, Sinv = hg_sqrt(HG, form)
    if rotate_out_on:
        W2 = rotate_out(W1, S, form, t)
    else:
        W2 = form_matmul(S, form, W1)
    H, lam = damped(HX2, damp)
    if order == "trace":
        sw = sweep_trace_order(W2, H, bits, group, block, search)
        R = sw["R_perm"]
    else:
        R = inverse_upper_factor(H)
        sw = (sweep_blocked(W2, R, bits, group, block, search=search) if mode == "blocked"
              else sweep_plain(W2, R, bits, group))
    out = {"HX": HX, "W1": W1, "HX2": HX2, "S": S, "Sinv": Sinv, "W2": W2, "lam": lam, "R": R,
           "score": sensitivity(HX, HG, form), "words": pack(sw["codes"], bits) if (i * bits) % 32 == 0 else None, **sw}
    if verify:
        if rotate_in and rotate_out_on:
            What = unrotate(sw["Q"], s, t, Sinv, form)
        else:
            A = form_matmul(Sinv, form, sw["Q"] if not rotate_out_on else _unrot(sw["Q"], t, axis=0))
            What = _unrot(A, s, axis=1) if rotate_in else A
        out["What"] = What
        out["loss"] = kfac_loss(W, What, HX, HG, form)
        out["loss_rot"] = float(rotated_loss(W2, sw["Q"], HX2).sum())
    return out
