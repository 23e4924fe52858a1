"""Comparison rules between the GPU path and the float64 oracle (test helpers).

Codes: rows are independent given R, so a rounding flip at a near-tie only cascades along its own
row. Each row is walked in sweep order; where the codes differ at a position whose oracle tie
distance is <= TIE (1e-4 grid steps), the row is replayed in the oracle with the GPU's code forced
there, and the walk continues. After replay every code, and every packed word, must match
bit-exactly; a difference at a position with tie distance > TIE is a failure.
"""
from __future__ import annotations

import numpy as np

from oracle import kronq as kq

TIE = 1e-4


def gpu_words_to_codes(words: np.ndarray, bits: int, i: int) -> np.ndarray:
    return kq.unpack(words.view(np.uint32), bits, i)


def replay_compare(gpu_codes: np.ndarray, W2: np.ndarray, R: np.ndarray, bits: int, group: int, block: int,
                   rows=None, tie: float = TIE, max_replays_per_row: int = 64, search: int = 0,
                   gpu_scale: np.ndarray | None = None) -> dict:
    """Compare GPU codes with the oracle sweep on W2 / R (float64), replaying near-tie flips.

    ``rows``: row indices of W2 / gpu_codes to check (all by default). W2 and gpu_codes are indexed by
    the same row numbers. The oracle first sweeps all those rows at once (rows are independent given
    R); only rows whose codes differ are then walked one by one with replays. Returns counts and the
    oracle codes / outputs after replay for those rows. With ``search`` the grids are chosen by the
    Hessian-aware search; ``gpu_scale`` (rows x groups) replays the GPU's candidate at every grid, and
    the candidates' objectives are returned so that the caller can check that choice against the
    oracle's minimum."""
    o, i = gpu_codes.shape
    rows = np.arange(o) if rows is None else np.asarray(rows)
    out = {"replays": 0, "fail": [], "codes": {}, "Q": {}, "row_loss": {}, "mu": {}, "scale": {}, "chosen": {},
           "objectives": {}, "delta": {}, "replayed_rows": []}

    def keep(r, res, k):
        out["codes"][int(r)] = res["codes"][k]
        out["Q"][int(r)] = res["Q"][k]
        out["row_loss"][int(r)] = res["row_loss"][k]
        out["mu"][int(r)] = res["mu"][k]
        out["scale"][int(r)] = res["scale"][k]
        out["delta"][int(r)] = res["delta"][k]
        if search:
            out["chosen"][int(r)] = res["chosen"][k]
            out["objectives"][int(r)] = res["objectives"][k]

    ns_all = None if gpu_scale is None else np.asarray(gpu_scale, np.float64)[rows]
    first = kq.sweep_blocked(W2[rows], R, bits, group, block, search=search, near_scale=ns_all)
    for k, r in enumerate(rows):
        if np.array_equal(first["codes"][k], gpu_codes[r]):
            keep(r, first, k)
            continue
        out["replayed_rows"].append(int(r))
        w = W2[r:r + 1]
        g = gpu_codes[r]
        fm = np.zeros((1, i), bool)
        fc = np.zeros((1, i), np.int64)
        n_rep = 0
        res = None
        while True:
            ns = None if gpu_scale is None else np.asarray(gpu_scale, np.float64)[r:r + 1]
            res = kq.sweep_blocked(w, R, bits, group, block, force_mask=fm, force_codes=fc, search=search,
                                   near_scale=ns)
            c = res["codes"][0]
            diff = np.nonzero(c != g)[0]
            if diff.size == 0:
                break
            j = diff[0]
            d = res["delta"][0, j]
            if d > tie or n_rep >= max_replays_per_row:
                out["fail"].append((int(r), int(j), float(d), int(c[j]), int(g[j])))
                break
            fm[0, j] = True
            fc[0, j] = g[j]
            n_rep += 1
        out["replays"] += n_rep
        keep(r, res, 0)
    return out


def stack_rows(cmp: dict, key: str, rows) -> np.ndarray:
    return np.stack([cmp[key][int(r)] for r in rows])


def grid_steps(gpu_mu: np.ndarray, gpu_scale: np.ndarray, or_mu: np.ndarray, or_scale: np.ndarray, bits: int):
    """Differences of the grid parameters measured in grid steps of the oracle's grid: |d mu| / s and
    (2^b - 1) |d s| / s, the largest shift they cause in a pre-rounding value u = (w - mu) / s with u in
    [0, 2^b - 1]. Groups with s = 0 (every value equal) must match exactly and are left out."""
    L = 2 ** bits - 1
    or_scale = np.asarray(or_scale, np.float64)
    pos = or_scale > 0
    dmu = np.abs(np.asarray(gpu_mu, np.float64) - or_mu)[pos] / or_scale[pos]
    ds = L * np.abs(np.asarray(gpu_scale, np.float64) - or_scale)[pos] / or_scale[pos]
    return (float(dmu.max()) if dmu.size else 0.0), (float(ds.max()) if ds.size else 0.0)


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def hx_tol(n: int) -> float:
    """Relative Frobenius bound for H_X from bf16 inputs over n tokens. Each 64-token stage sums two
    exact 32-product matrix-core results in fp32 (two roundings, of magnitude u |s_32| and u |s_64|,
    u = 2^-24) before the fp64 accumulation, so the error grows like sqrt(n / 64) while H grows like
    n: about 3 u sqrt(32 / n) relative, bounded here with a factor of ~5 to spare. Far inside the
    1e-5 relative bound on H_X for every n >= 32."""
    return 1e-6 * (32.0 / n) ** 0.5



def matvec_error_scale(words: np.ndarray, mu: np.ndarray, scale: np.ndarray, bits: int, group: int, s: np.ndarray,
                       Sinv: np.ndarray, form: str, X: np.ndarray) -> np.ndarray:
    """Per-token scale of the fp32 rounding error of the factored product y = S^{-1} V^T Q'' U^T x:
    ||S^{-1}||_2 * || |Q''| |x'| ||_2 with x' = U^T x. The sums over the codes carry an error of at
    most a few ulps of |Q''| |x'| per element; the orthogonal transforms keep 2-norms, and S^{-1}
    can grow them by at most its spectral norm."""
    X = np.asarray(X, np.float64)
    i = X.shape[1]
    Q2 = kq.dequantize(kq.unpack(words, bits, i), np.asarray(mu, np.float64), np.asarray(scale, np.float64), group)
    Xr = kq.rotate_in_weights(X, s)                     # rows x' = U^T x
    Z = np.abs(Xr) @ np.abs(Q2).T                       # n x o
    if form == "diag":
        nrm = np.max(np.abs(Sinv))
    elif form == "block":
        nrm = max(np.linalg.norm(b, 2) for b in np.asarray(Sinv, np.float64))
    else:
        nrm = np.linalg.norm(np.asarray(Sinv, np.float64), 2)
    return nrm * np.linalg.norm(Z, axis=1)
