"""Pins of the float64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: an explicit
Kronecker product, integer identities of Hadamard matrices, invariants of
function-preserving transforms, a textbook Optimal Brain Surgeon sweep, brute
force over tiny code spaces, a closed-form expectation, or hand-worked values.
"""
import json
import os

import numpy as np
import pytest

from oracle import alloc, hadamard as hd, kronq as kq

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def spd(rng, d, n=None, spread=1.0):
    n = n or 4 * d
    G = rng.standard_normal((n, d)) * np.exp(spread * rng.standard_normal(d))
    return G.T @ G / n


def signs(rng, d):
    return (rng.integers(0, 2, d) * 2 - 1).astype(np.int8)


# ----------------------------------------------------------------------------- P1
@pytest.mark.parametrize("o,i", [(1, 1), (2, 3), (4, 5), (6, 6), (5, 2)])
def test_p1_kronecker_loss_identity(o, i):
    """vec(dW)^T (H_X (x) H_G) vec(dW) = tr(H_G dW H_X dW^T) with column-stacking vec;
    row-stacking pairs with H_G (x) H_X (review page, Background: H ~ H_X (x) H_G)."""
    rng = np.random.default_rng(o * 10 + i)
    HX, HG = spd(rng, i), spd(rng, o)
    W = rng.standard_normal((o, i))
    What = W + rng.standard_normal((o, i))
    dW = What - W
    vc = dW.flatten(order="F")
    vr = dW.flatten(order="C")
    ref_col = vc @ np.kron(HX, HG) @ vc
    ref_row = vr @ np.kron(HG, HX) @ vr
    got = kq.kfac_loss(W, What, HX, HG, "full")
    assert np.isclose(got, ref_col, rtol=1e-12)
    assert np.isclose(got, ref_row, rtol=1e-12)
    # the diagonal and block forms agree with the dense matrix
    hd_ = np.abs(rng.standard_normal(o)) + 0.1
    assert np.isclose(kq.kfac_loss(W, What, HX, hd_, "diag"), vc @ np.kron(HX, np.diag(hd_)) @ vc, rtol=1e-12)


# ----------------------------------------------------------------------------- P2
@pytest.mark.parametrize("d", [1, 2, 4, 8, 64, 256, 1024, 12, 20, 28, 40, 108, 344, 56, 216])
def test_p2_hadamard_orthogonality_and_fast_apply(d):
    H = hd.hadamard(d)
    assert set(np.unique(H)) <= {-1, 1}
    assert np.array_equal(H @ H.T, d * np.eye(d, dtype=np.int64))
    x = np.random.default_rng(d).standard_normal((3, d))
    assert np.allclose(hd.apply(x), x @ H.T, atol=1e-9)
    assert np.allclose(hd.apply(x, transpose=True), x @ H, atol=1e-9)
    assert np.allclose(hd.apply(x.T, axis=0), H @ x.T, atol=1e-9)


def test_p2_config_dimensions_decompose():
    want = {256: (1, 256), 4096: (1, 4096), 5120: (20, 256), 13824: (108, 128),
            28672: (28, 1024), 11008: (344, 32), 8192: (1, 8192)}
    for d, mk in want.items():
        assert hd.decompose(d) == mk
    for m in (20, 28, 108, 344):
        P = hd.paley(m)
        assert np.array_equal(P @ P.T, m * np.eye(m, dtype=np.int64))
    with pytest.raises(ValueError):
        hd.decompose(3 * 5 * 17)   # no admissible order


def test_p2_finite_field_tables():
    # quadratic residues mod 7 are {1, 2, 4}
    chi7 = hd.quadratic_character(7)
    assert [i for i in range(7) if chi7[i] == 1] == [1, 2, 4]
    for q in (19, 27, 107, 343):
        chi = hd.quadratic_character(q)
        assert chi[0] == 0 and (chi == 1).sum() == (q - 1) // 2 and (chi == -1).sum() == (q - 1) // 2
        minus_one = hd.gf_sub(q, 0, 1)
        assert chi[minus_one] == -1      # q = 3 mod 4
    # GF(27): multiplicative group is cyclic of order 26 and chi is multiplicative
    _, _, mul = hd._gf_elements(27)
    chi = hd.quadratic_character(27)
    orders = []
    for g in range(1, 27):
        x, k = g, 1
        while x != 1:
            x, k = mul(x, g), k + 1
        orders.append(k)
    assert max(orders) == 26
    for a in range(1, 27):
        for b in range(1, 27):
            assert chi[mul(a, b)] == chi[a] * chi[b]


# ----------------------------------------------------------------------------- P3
@pytest.mark.parametrize("o,i", [(8, 12), (20, 16), (16, 20)])
def test_p3_rotations_preserve_layer_output(o, i):
    """(XU)(WU)^T = XW^T and S^{-1} V^T (W'' U^T x) = W x (Hessian-guided PTQ page,
    Background: function-preserving transforms (XT)(T^{-1}W) = Z)."""
    rng = np.random.default_rng(o + 3 * i)
    X = rng.standard_normal((30, i))
    W = rng.standard_normal((o, i))
    s, t = signs(rng, i), signs(rng, o)
    U = kq.rotation_matrix(s)
    assert np.allclose(U @ U.T, np.eye(i), atol=1e-12)
    W1 = kq.rotate_in_weights(W, s)
    assert np.allclose(W1, W @ U, atol=1e-12)
    assert np.allclose((X @ U) @ W1.T, X @ W.T, atol=1e-10)
    HX = X.T @ X / 30
    HX2 = kq.rotate_in_hessian(HX, s)
    assert np.allclose(HX2, U.T @ HX @ U, atol=1e-10)
    assert np.isclose(np.trace(HX2), np.trace(HX))
    assert np.allclose(np.linalg.eigvalsh(HX2), np.linalg.eigvalsh(HX), atol=1e-9)
    HG = spd(rng, o)
    S, Si = kq.hg_sqrt(HG, "full")
    W2 = kq.rotate_out(W1, S, "full", t)
    V = np.diag(t.astype(float)) @ hd.hadamard(o).T / np.sqrt(o)       # V = H_o D_t / sqrt(o) -> V^T
    assert np.allclose(W2, V.T @ S @ W1, atol=1e-10)
    What = kq.unrotate(W2, s, t, Si, "full")
    assert np.allclose(What, W, atol=1e-9)
    x = rng.standard_normal(i)
    assert np.allclose(Si @ V @ (W2 @ (U.T @ x)), W @ x, atol=1e-9)


# ----------------------------------------------------------------------------- P4
def test_p4_square_root_and_loss_in_both_coordinates():
    rng = np.random.default_rng(4)
    o, i = 12, 16
    HG = spd(rng, o, spread=2.0)
    S, Si = kq.hg_sqrt(HG, "full")
    assert np.allclose(S, S.T) and np.all(np.linalg.eigvalsh(S) > 0)
    assert np.allclose(S @ S, HG, atol=1e-10 * np.abs(HG).max())
    assert np.allclose(S @ Si, np.eye(o), atol=1e-9)
    assert np.allclose(Si @ HG @ Si, np.eye(o), atol=1e-8)
    hdg = np.abs(rng.standard_normal(o)) + 0.01
    Sd, Sdi = kq.hg_sqrt(hdg, "diag")
    assert np.array_equal(Sd, np.sqrt(hdg))
    blocks = np.stack([spd(rng, 4) for _ in range(3)])
    Sb, Sbi = kq.hg_sqrt(blocks, "block")
    for k in range(3):
        assert np.allclose(Sb[k] @ Sb[k], blocks[k], atol=1e-10)
    # loss in original coordinates = loss in rotated coordinates, every H_G form
    X = rng.standard_normal((64, i))
    W = rng.standard_normal((o, i)) * 0.02
    s, t = signs(rng, i), signs(rng, o)
    for form, hg in (("full", HG), ("diag", hdg), ("block", blocks)):
        r = kq.quantize_layer(X, W, hg, form, s, t, bits=3, group=0, block=8)
        assert np.isclose(r["loss"], r["loss_rot"], rtol=1e-9)


# ----------------------------------------------------------------------------- P5
@pytest.mark.parametrize("bits,group", [(2, 0), (3, 0), (4, 0), (3, 4), (2, 8)])
def test_p5_cholesky_sweep_equals_naive_obs(bits, group):
    rng = np.random.default_rng(5 + bits + group)
    o, i = 6, 16
    H, _ = kq.damped(spd(rng, i, spread=1.0))
    W = rng.standard_normal((o, i))
    R = kq.inverse_upper_factor(H)
    assert np.allclose(np.triu(R), R) and np.all(np.diag(R) > 0)
    assert np.allclose(R.T @ R @ H, np.eye(i), atol=1e-9)
    a = kq.sweep_plain(W, R, bits, group)
    b = kq.sweep_obs_naive(W, H, bits, group)
    assert np.array_equal(a["codes"], b["codes"])
    assert np.allclose(a["Q"], b["Q"], atol=1e-10)
    assert np.allclose(a["row_loss"], b["row_loss"], rtol=1e-9)
    for blk in (4, 8, 16):
        if group and (blk % group) and (group % blk):
            continue
        c = kq.sweep_blocked(W, R, bits, group, block=blk)
        assert np.array_equal(a["codes"], c["codes"])
        assert np.allclose(a["Q"], c["Q"], atol=1e-10)
        assert np.allclose(a["mu"], c["mu"], atol=1e-12) and np.allclose(a["scale"], c["scale"], atol=1e-12)


def test_p5_upper_factor_closed_form_2x2():
    a, b, c = 3.0, 1.2, 2.0
    det = a * c - b * b
    r00 = np.sqrt(c / det)
    r01 = (-b / det) / r00
    r11 = np.sqrt(a / det - r01 ** 2)
    R = kq.inverse_upper_factor(np.array([[a, b], [b, c]]))
    assert np.allclose(R, [[r00, r01], [0.0, r11]], atol=1e-14)


# ----------------------------------------------------------------------------- P6
def test_p6_row_loss_is_damped_quadratic_form():
    rng = np.random.default_rng(6)
    o, i = 5, 32
    H, _ = kq.damped(spd(rng, i, spread=1.5))
    W = rng.standard_normal((o, i))
    r = kq.sweep_blocked(W, kq.inverse_upper_factor(H), 3, 8, block=16)
    dW = r["Q"] - W
    assert np.allclose(r["row_loss"], np.einsum("ri,ij,rj->r", dW, H, dW), rtol=1e-9)


# ----------------------------------------------------------------------------- P7 / P9 (continuous remainder)
@pytest.mark.parametrize("stop", [1, 3, 6])
@pytest.mark.parametrize("hg_kind", ["identity", "full"])
def test_p7_remainder_minimises_kronecker_loss_for_any_HG(stop, hg_kind):
    """After quantizing the first ``stop`` columns, the still-continuous weights minimise
    vec(dW)^T (H (x) H_G) vec(dW) given the quantized ones, whatever H_G is: the H_G factor
    cancels from the update (review page, Method / Key idea; Hessian-guided PTQ page: with GPTQ
    rounding only the first Kronecker factor determines the corrections)."""
    rng = np.random.default_rng(7 + stop)
    o, i = 3, 7
    H, _ = kq.damped(spd(rng, i, spread=1.0))
    HG = np.eye(o) if hg_kind == "identity" else spd(rng, o, spread=1.5)
    W = rng.standard_normal((o, i))
    part = kq.sweep_plain(W, kq.inverse_upper_factor(H), 3, 0, stop=stop)["Q"]
    dW = part - W
    K = np.kron(H, HG)                                   # column-stacking index = col * o + row
    fixed = np.zeros((o, i), bool)
    fixed[:, :stop] = True
    fx = fixed.flatten(order="F")
    v = dW.flatten(order="F")
    opt = -np.linalg.solve(K[~fx][:, ~fx], K[~fx][:, fx] @ v[fx])
    assert np.allclose(v[~fx], opt, atol=1e-10)


# ----------------------------------------------------------------------------- P8
def test_p8_identity_HG_without_rotations_is_gptq_on_W():
    rng = np.random.default_rng(8)
    o, i = 6, 32
    X = rng.standard_normal((50, i)) * np.exp(rng.standard_normal(i))
    W = rng.standard_normal((o, i))
    r = kq.quantize_layer(X, W, np.ones(o), "diag", None, None, 3, 0, block=8,
                          rotate_in=False, rotate_out_on=False)
    H, _ = kq.damped(X.T @ X / 50)
    g = kq.sweep_obs_naive(W, H, 3, 0)
    assert np.array_equal(r["codes"], g["codes"])
    assert np.allclose(r["What"], g["Q"], atol=1e-10)


def test_p8_diagonal_HG_without_V_gives_gptq_codes_on_WU():
    """Per-row grids are scale-equivariant, and the sweep is row-independent and linear."""
    rng = np.random.default_rng(81)
    o, i = 8, 32
    X = rng.standard_normal((64, i))
    W = rng.standard_normal((o, i))
    s = signs(rng, i)
    h = 10 ** rng.uniform(-2, 2, o)
    r = kq.quantize_layer(X, W, h, "diag", s, None, 3, 0, block=8, rotate_out_on=False)
    H, _ = kq.damped(kq.rotate_in_hessian(X.T @ X / 64, s))
    g = kq.sweep_obs_naive(kq.rotate_in_weights(W, s), H, 3, 0)
    assert np.array_equal(r["codes"], g["codes"])


# ----------------------------------------------------------------------------- P9
def test_p9_diagonal_hessian_is_round_to_nearest():
    rng = np.random.default_rng(9)
    o, i = 4, 32
    H = np.diag(np.exp(rng.standard_normal(i)))
    W = rng.standard_normal((o, i))
    r = kq.sweep_plain(W, kq.inverse_upper_factor(H), 3, 8)
    mu, sc = kq.grid_params(W.reshape(o, i // 8, 8), 3)
    rtn = np.clip(np.rint((W.reshape(o, i // 8, 8) - mu[..., None]) / sc[..., None]), 0, 7).reshape(o, i)
    assert np.array_equal(r["codes"], rtn.astype(np.int64))


@pytest.mark.parametrize("i", [1, 2, 4, 6])
def test_p9_brute_force_lower_bounds_gptq(i):
    rng = np.random.default_rng(90 + i)
    o, bits = 2, 2
    H, _ = kq.damped(spd(rng, i, n=3 * i + 2, spread=1.0))
    W = rng.standard_normal((o, i))
    r = kq.sweep_plain(W, kq.inverse_upper_factor(H), bits, 0)
    mu, sc = kq.grid_params(W, bits)
    L = 2 ** bits
    grids = np.array(np.meshgrid(*[np.arange(L)] * i, indexing="ij")).reshape(i, -1).T
    for row in range(o):
        cand = mu[row] + sc[row] * grids
        d = cand - W[row]
        best = np.min(np.einsum("ki,ij,kj->k", d, H, d))
        g = r["row_loss"][row]
        assert best <= g * (1 + 1e-12) + 1e-15
        if i == 1:
            assert np.isclose(best, g, rtol=1e-12)


# ----------------------------------------------------------------------------- P10
def test_p10_score_is_expected_loss_coefficient():
    """E[tr(H_G dW H_X dW^T)] = sigma^2 tr(H_G) tr(H_X) for iid zero-mean errors; for uniform rounding
    errors of step d, sigma^2 = d^2 / 12 (Hessian-guided PTQ page, appendix: rounding-noise model)."""
    rng = np.random.default_rng(10)
    o, i, n = 5, 6, 200000
    HX, HG = spd(rng, i), spd(rng, o)
    d = 0.3
    dW = rng.uniform(-d / 2, d / 2, size=(n, o, i))
    vals = np.einsum("ab,nbi,ij,naj->n", HG, dW, HX, dW)
    score = kq.sensitivity(HX, HG, "full")
    assert abs(vals.mean() / (d * d / 12 * score) - 1) < 0.01
    X = rng.standard_normal((40, i))
    assert np.isclose(kq.sensitivity(X.T @ X / 40, np.eye(o), "full"), o * (X ** 2).sum() / 40)


# ----------------------------------------------------------------------------- P11
def test_p11_allocation():
    # equal scores and sizes -> uniform 3 bits, budget met exactly
    b = alloc.allocate(np.ones(7), np.full(7, 100), 3.0)
    assert np.array_equal(b, np.full(7, 3))
    # budget never exceeded; no single further upgrade fits
    rng = np.random.default_rng(11)
    for _ in range(20):
        sc = np.exp(3 * rng.standard_normal(9))
        sz = rng.choice([16, 16, 16, 16, 43, 43, 43], 9)
        b = alloc.allocate(sc, sz, 3.0)
        assert np.dot(b, sz) <= 3.0 * sz.sum()
        spare = 3.0 * sz.sum() - np.dot(b, sz)
        assert all(b[k] == 4 or sz[k] > spare for k in range(9))
        ex = alloc.allocate_exact(sc, sz, 3.0)
        assert alloc.expected_loss(sc, ex) <= alloc.expected_loss(sc, b) + 1e-12
    # q, k, v share H_X: ordered by tr(H_G)
    b = alloc.allocate([1.0, 5.0, 2.0, 1.0], [10, 10, 10, 10], 2.5)
    assert b[1] >= b[2] >= b[0] and b[1] >= b[2] >= b[3]


# ----------------------------------------------------------------------------- P12 (soft)
def test_p12_bidirectional_rotation_flattens_weight_magnitudes():
    """Review page, "Where this paper sits" (Appendix D): rotations on both axes flatten the
    per-channel spread of weight magnitudes."""
    rng = np.random.default_rng(12)
    o, i = 64, 128
    W = rng.standard_normal((o, i)) * 0.02
    W[:, rng.choice(i, 3, replace=False)] *= 30
    W[rng.choice(o, 2, replace=False), :] *= 15
    s, t = signs(rng, i), signs(rng, o)

    def cv(v):
        return v.std() / v.mean()

    W2 = kq.rotate_out(kq.rotate_in_weights(W, s), np.ones(o), "diag", t)
    assert cv(np.linalg.norm(W2, axis=0)) < 0.5 * cv(np.linalg.norm(W, axis=0))
    assert cv(np.linalg.norm(W2, axis=1)) < 0.5 * cv(np.linalg.norm(W, axis=1))


# ----------------------------------------------------------------------------- grid, packing
def test_grid_worked_example():
    with open(os.path.join(GOLD, "grid_worked.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        v = np.array(case["values"], dtype=np.float64)
        mu, s = kq.grid_params(v[None, :], case["bits"])
        assert np.isclose(mu[0], case["mu"]) and np.isclose(s[0], case["step"])
        q, deq, _ = kq.quantize(np.array(case["probe"], np.float64), mu[0], s[0], case["bits"])
        assert q.tolist() == case["codes"]


def test_pack_matches_big_integer_bitstream():
    rng = np.random.default_rng(13)
    for bits in (2, 3, 4, 8):
        i = 32 * 3
        codes = rng.integers(0, 2 ** bits, size=(3, i))
        words = kq.pack(codes, bits)
        for r in range(3):
            big = 0
            for j in range(i):
                big |= int(codes[r, j]) << (bits * j)
            want = [(big >> (32 * w)) & 0xFFFFFFFF for w in range(i * bits // 32)]
            assert words[r].tolist() == want
        assert np.array_equal(kq.unpack(words, bits, i), codes)
    # hand-worked: 3-bit codes 1..7,0 then 5 -> first word
    c = np.zeros((1, 32), np.int64)
    c[0, :9] = [1, 2, 3, 4, 5, 6, 7, 0, 5]
    w0 = 1 | 2 << 3 | 3 << 6 | 4 << 9 | 5 << 12 | 6 << 15 | 7 << 18 | 0 << 21 | 5 << 24
    assert int(kq.pack(c, 3)[0, 0]) == w0


# ----------------------------------------------------------------------------- P13
@pytest.mark.parametrize("form", ["diag", "full"])
def test_p13_matvec_zero_codes_closed_form(form):
    """Inference-side product (KronQ review page, Limitations (3)) with every code 0 and mu = 1
    (one group per row): Q'' = 1 1^T, and with a Sylvester Hadamard (first row and column all
    ones) U 1 = sqrt(i) s_0 e_0 and V^T 1 = sqrt(o) t_0 e_0, so W^ x = sqrt(o i) s_0 t_0 x_0 S^{-1} e_0."""
    rng = np.random.default_rng(21)
    o, i, bits, n = 16, 64, 4, 3
    s, t = signs(rng, i), signs(rng, o)
    Si = np.exp(rng.standard_normal(o)) if form == "diag" else spd(rng, o)
    words = np.zeros((o, i * bits // 32), np.uint32)
    mu = np.ones((o, 1))
    sc = rng.random((o, 1))
    X = rng.standard_normal((n, i))
    Y = kq.matvec_quantized(words, mu, sc, bits, 0, s, t, Si, form, X)
    e0 = np.zeros(o)
    e0[0] = 1.0
    col0 = Si * e0 if form == "diag" else Si[:, 0]       # S^{-1} e_0
    want = np.sqrt(o * i) * s[0] * t[0] * X[:, :1] * col0[None, :]
    assert np.allclose(Y, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("bits,group", [(3, 0), (2, 32), (5, 32)])
def test_p13_matvec_brute_force(bits, group):
    """The same product by brute force on a tiny layer: codes read bit by bit from the words as
    one big integer per row, w = mu + s q per element, dense Sylvester matrices from scipy, and
    y = S^{-1} V^T Q'' U^T x as plain dense products."""
    from scipy.linalg import hadamard as sylvester
    rng = np.random.default_rng(bits * 7 + group)
    o, i, n = 8, 64, 2
    words = rng.integers(0, 2 ** 32, size=(o, i * bits // 32), dtype=np.uint64).astype(np.uint32)
    g = group if group else i
    mu = rng.standard_normal((o, i // g))
    sc = rng.random((o, i // g))
    s, t = signs(rng, i), signs(rng, o)
    Si = spd(rng, o)
    X = rng.standard_normal((n, i))
    Q = np.zeros((o, i))
    for r in range(o):
        big = 0
        for k, wd in enumerate(words[r].tolist()):
            big |= int(wd) << (32 * k)
        for c in range(i):
            q = (big >> (bits * c)) & ((1 << bits) - 1)
            Q[r, c] = mu[r, c // g] + sc[r, c // g] * q
    U = np.diag(s.astype(float)) @ sylvester(i).T / np.sqrt(i)
    V = sylvester(o) @ np.diag(t.astype(float)) / np.sqrt(o)
    What = Si @ V.T @ Q @ U.T
    Y = kq.matvec_quantized(words, mu, sc, bits, group, s, t, Si, "full", X)
    assert np.allclose(Y, X @ What.T, rtol=1e-11, atol=1e-11)


# ----------------------------------------------------------------------------- P14
def test_p14_lowrank_diagonal_closed_form():
    """H = diag(h) with Omega = the first k unit vectors: the range is exactly those coordinates for
    any number of power steps, so H^ = diag(h_1..h_k, sigma, .., sigma), sigma = mean of the rest."""
    o, k, n = 12, 4, 12
    h = np.linspace(5.0, 0.5, o)
    G = np.zeros((n, o))
    G[np.arange(o), np.arange(o)] = np.sqrt(n * h)
    omega = np.eye(o)[:, :k]
    for q in (0, 2):
        r = kq.hg_lowrank(G, k, q, omega)
        sig = h[k:].mean()
        assert np.isclose(r["sigma"], sig, rtol=1e-13)
        want = np.diag(np.concatenate([h[:k], np.full(o - k, sig)]))
        assert np.allclose(r["Hhat"], want, atol=1e-12)
        assert np.allclose(r["S"], np.sqrt(want), atol=1e-12)
        assert np.allclose(r["Sinv"] @ r["S"], np.eye(o), atol=1e-12)


def test_p14_lowrank_exact_rank_and_trace():
    """G of rank k: H^ = H (sigma = 0) for a generic Omega; for any G the trace is kept and S^2 = H^."""
    rng = np.random.default_rng(5)
    o, k, n = 40, 6, 60
    G = rng.standard_normal((n, k)) @ rng.standard_normal((k, o))
    r = kq.hg_lowrank(G, k, 1, rng.standard_normal((o, k)))
    assert abs(r["sigma"]) < 1e-12 * r["trH"]
    assert np.allclose(r["Hhat"], r["H"], atol=1e-10 * np.abs(r["H"]).max())
    G = rng.standard_normal((n, o)) * np.exp(rng.standard_normal(o))
    r = kq.hg_lowrank(G, k, 2, rng.standard_normal((o, k)))
    assert np.isclose(np.trace(r["Hhat"]), np.trace(r["H"]), rtol=1e-12)
    assert np.allclose(r["S"] @ r["S"], r["Hhat"], atol=1e-10 * np.abs(r["Hhat"]).max())
    assert np.allclose(r["Sinv"] @ r["S"], np.eye(o), atol=1e-9)
    # on the captured subspace H^ acts as H: Q^T H^ Q = Q^T H Q
    Q = r["Q"]
    assert np.allclose(Q.T @ r["Hhat"] @ Q, Q.T @ r["H"] @ Q, atol=1e-10 * np.abs(r["H"]).max())
    # a full-rank k = o - 1 capture of the top eigenspace with many power steps approaches H
    w, V = np.linalg.eigh(r["H"])
    r2 = kq.hg_lowrank(G, o - 1, 30, rng.standard_normal((o, o - 1)))
    assert np.isclose(r2["sigma"], w[0], rtol=1e-6)


def test_p14_forms_are_slices():
    rng = np.random.default_rng(2)
    H = spd(rng, 8)
    assert np.array_equal(kq.hg_forms(H, "diag"), np.diag(H))
    blocks = kq.hg_forms(H, "block", 4)
    assert blocks.shape == (2, 4, 4) and np.array_equal(blocks[1], H[4:, 4:])
    assert np.array_equal(kq.hg_forms(H, "full"), H)


# ----------------------------------------------------------------------------- P15
def test_p15_grid_search_brute_force_and_bound():
    """Hessian-aware grid: the argmin over the candidates by explicit scalar loops (round half to
    even written out), the min-max grid as the alpha = 1 candidate, and a weighted error never above
    the min-max grid's."""
    rng = np.random.default_rng(9)
    bits, M = 3, 41
    L = 2 ** bits - 1
    v = rng.standard_normal((5, 6))
    d = np.exp(rng.standard_normal(6))
    mu, s, idx, obj = kq.grid_search(v, d, bits, M)
    mu1, s1 = kq.grid_params(v, bits)
    assert np.allclose(obj[:, -1], [np.sum(d * (v[r] - kq.quantize(v[r], mu1[r], s1[r], bits)[1]) ** 2)
                                    for r in range(5)], rtol=1e-12)
    assert np.all(obj[np.arange(5), idx] <= obj[:, -1])

    def rne(x):
        f = np.floor(x)
        frac = x - f
        return f + 1 if frac > 0.5 else f if frac < 0.5 else (f if f % 2 == 0 else f + 1)
    for r in range(5):
        lo, hi = v[r].min(), v[r].max()
        best, bi = None, None
        for m in range(M):
            a = 0.5 + 0.5 * m / (M - 1)
            st = 2 * a * (hi - lo) / 2 / L
            off = (lo + hi) / 2 - a * (hi - lo) / 2
            e = 0.0
            for c in range(6):
                q = min(max(rne((v[r, c] - off) / st), 0), L)
                e += d[c] * (v[r, c] - (off + st * q)) ** 2
            if best is None or e < best:
                best, bi = e, m
        assert bi == idx[r] and np.isclose(best, obj[r, idx[r]], rtol=1e-12)


def test_p15_grid_search_special_cases():
    """Values exactly on the min-max grid keep it (zero error, every smaller range errs); a
    low-weight outlier is clipped (a smaller range wins); one candidate is min-max; the sweep with
    one candidate equals the plain sweep."""
    bits, L = 2, 3
    v = np.array([[0.0, 1.0, 2.0, 3.0, 1.0, 2.0]])
    mu, s, idx, obj = kq.grid_search(v, np.ones(6), bits, 500)
    assert idx[0] == 499 and obj[0, 499] == 0.0 and np.all(obj[0, :499] > 0)
    v = np.array([[0.0, 0.1, 0.2, 0.3, 0.15, 10.0]])
    d = np.array([1.0, 1.0, 1.0, 1.0, 1.0, 1e-9])
    mu, s, idx, obj = kq.grid_search(v, d, bits, 500)
    assert idx[0] < 499 and obj[0, idx[0]] < obj[0, 499]
    rng = np.random.default_rng(1)
    W = rng.standard_normal((6, 256))
    R = np.triu(rng.standard_normal((256, 256)) * 0.01) + np.eye(256)
    a = kq.sweep_blocked(W, R, 3, 32, 128)
    b = kq.sweep_blocked(W, R, 3, 32, 128, search=1)
    assert np.array_equal(a["codes"], b["codes"]) and np.allclose(a["Q"], b["Q"], atol=1e-12)


# ----------------------------------------------------------------------------- P16
def test_p16_trace_order():
    """Trace-ordered blocks: the order sorts block traces descending (stable); blocks already in that
    order give the plain sweep; two blocks in ascending order equal the plain sweep on hand-swapped
    inputs, swapped back; the row loss equals dW (H_X' + lambda I) dW^T in natural coordinates."""
    rng = np.random.default_rng(12)
    d = np.array([1.0, 5.0, 3.0, 5.0])
    H = np.diag(np.repeat(d, 2))
    assert list(kq.block_trace_order(H, 2)) == [1, 3, 2, 0]
    i, o, bits, g = 256, 5, 3, 64
    A = rng.standard_normal((2 * i, i))
    Hx0 = A.T @ A / (2 * i)
    D = np.ones(i)
    D[:128] = 2.0                           # congruence keeps H SPD; first block's trace x4: identity order
    Hx = Hx0 * np.outer(D, D)
    H, lam = kq.damped(Hx)
    W = rng.standard_normal((o, i))
    a = kq.sweep_trace_order(W, H, bits, g)
    assert list(a["order"]) == [0, 1]
    b = kq.sweep_blocked(W, kq.inverse_upper_factor(H), bits, g)
    assert np.array_equal(a["codes"], b["codes"]) and np.allclose(a["Q"], b["Q"], atol=1e-12)
    D[:128] = 0.5                           # now the second block leads
    H2, _ = kq.damped(Hx0 * np.outer(D, D))
    c = kq.sweep_trace_order(W, H2, bits, g)
    assert list(c["order"]) == [1, 0]
    p = np.concatenate([np.arange(128, 256), np.arange(0, 128)])
    ref = kq.sweep_blocked(W[:, p], kq.inverse_upper_factor(H2[np.ix_(p, p)]), bits, g)
    assert np.array_equal(c["codes"][:, p], ref["codes"]) and np.allclose(c["Q"][:, p], ref["Q"], atol=1e-12)
    assert np.allclose(c["scale"], np.concatenate([ref["scale"][:, 2:], ref["scale"][:, :2]], axis=1))
    dW = W - c["Q"]
    assert np.allclose(np.einsum("ri,ij,rj->r", dW, H2, dW), c["row_loss"], rtol=1e-9)


# ----------------------------------------------------------------------------- P17
def test_p17_drift_target():
    """Input-drift target: no drift and no damping gives W back; without damping the residual
    splits exactly (W* is the least-squares fit of W X^T from X~); with damping the ridge gradient
    vanishes at W*. Parity of GPTAQ's own column-wise formula is unpinned (not on the pages)."""
    rng = np.random.default_rng(17)
    n, i, o = 300, 24, 7
    X = rng.standard_normal((n, i)) * np.exp(rng.standard_normal(i))
    Xt = X + 0.1 * rng.standard_normal((n, i))
    W = rng.standard_normal((o, i))
    assert np.allclose(kq.drift_target(W, X, X, damp=0.0)["W"], W, atol=1e-10)
    Ws = kq.drift_target(W, X, Xt, damp=0.0)["W"]
    V = W + rng.standard_normal((o, i))
    lhs = np.sum((V @ Xt.T - W @ X.T) ** 2)
    rhs = np.sum(((V - Ws) @ Xt.T) ** 2) + np.sum((Ws @ Xt.T - W @ X.T) ** 2)
    assert np.isclose(lhs, rhs, rtol=1e-10)
    d = kq.drift_target(W, X, Xt, damp=0.05)
    grad = (d["W"] @ Xt.T - W @ X.T) @ Xt + n * d["lam"] * d["W"]
    assert np.abs(grad).max() <= 1e-9 * np.abs(W @ X.T @ Xt).max()


def test_golden_regression_small_layer():
    """Stored oracle outputs of the small 256x256 workload (written by tests/golden/make_golden.py,
    which calls only the oracle) guard the oracle against accidental change."""
    import hashlib
    import synth
    with open(os.path.join(GOLD, "c1_oracle.json")) as f:
        g = json.load(f)
    sp = synth.CONFIGS["C1"]
    d = synth.layer_inputs(sp)
    r = kq.quantize_layer(synth.widen(d["X"], sp.x_dtype), synth.widen(d["W"], sp.w_dtype), d["HG"].astype(np.float64),
                          sp.hg_form, d["s"], d["t"], sp.bits, sp.group, sp.block, sp.damp)
    assert hashlib.sha256(r["words"].tobytes()).hexdigest() == g["words_sha256"]
    assert np.isclose(r["loss"], g["loss"], rtol=1e-9)
    assert np.isclose(r["score"], g["score"], rtol=1e-12)


# ----------------------------------------------------------------------------- P18: hand-worked values
def test_p18_hessian_hand_worked():
    """H_X = X^T X / n, the second moment of the calibration inputs over the token count (review page,
    Background: the input activation covariance as the layer-Hessian proxy). Worked by hand for two
    tokens x_1 = (1, 2), x_2 = (3, -1): X^T X = [[1 + 9, 2 - 3], [2 - 3, 4 + 1]] = [[10, -1], [-1, 5]],
    divided by n = 2. Dividing by n - 1, not dividing, or centring the tokens fails."""
    X = np.array([[1.0, 2.0], [3.0, -1.0]])
    assert np.array_equal(kq.hessian(X), np.array([[5.0, -0.5], [-0.5, 2.5]]))
    # three tokens, one channel: (4 + 1 + 16) / 3 = 7
    assert np.array_equal(kq.hessian(np.array([[2.0], [-1.0], [4.0]])), np.array([[7.0]]))
    # the input dtype is widened exactly: bf16-representable values give the same result
    assert kq.hessian(np.array([[0.5, 0.25]], dtype=np.float32)).dtype == np.float64


def test_p18_damping_hand_worked():
    """lambda = damp * mean(diag H) (GPTQ damping, 1 % of the average diagonal; the workloads' own
    statement for the smallest layer). H = diag(1, 2, 3, 6): mean diag = 3, so lambda = 0.03 at
    damp 0.01; 0.01 * max diag (0.06) or 0.01 * trace (0.12) fails. Only the diagonal moves."""
    H = np.diag([1.0, 2.0, 3.0, 6.0])
    Hd, lam = kq.damped(H)
    assert np.isclose(lam, 0.03, rtol=0, atol=1e-15)
    assert np.allclose(Hd, np.diag([1.03, 2.03, 3.03, 6.03]), rtol=0, atol=1e-15)
    A = np.array([[4.0, 1.0], [1.0, 2.0]])
    Ad, lam = kq.damped(A, 0.1)
    assert np.isclose(lam, 0.3, rtol=0, atol=1e-15)
    assert np.allclose(Ad, [[4.3, 1.0], [1.0, 2.3]], rtol=0, atol=1e-15)


def test_p18_trace_forms_hand_worked():
    """tr(H_G) in the three storage forms (review page, Method (2): the score tr(H_G) tr(H_X)). Diagonal
    (1, 2, 3): 6. Two blocks [[1, 5], [7, 2]] and [[3, 0], [0, 4]]: 1 + 2 + 3 + 4 = 10 (off-diagonal
    entries do not count). Full: the same matrix block-diagonal in dense form, 10."""
    assert kq.trace_form(np.array([1.0, 2.0, 3.0]), "diag") == 6.0
    blocks = np.array([[[1.0, 5.0], [7.0, 2.0]], [[3.0, 0.0], [0.0, 4.0]]])
    assert kq.trace_form(blocks, "block") == 10.0
    assert kq.trace_form(kq.form_dense(blocks, "block"), "full") == 10.0
    # the score: tr(H_G) = 1 + 3 = 4 and tr(H_X) = 5 + 2.5 = 7.5 for the two tokens above
    X = np.array([[1.0, 2.0], [3.0, -1.0]])
    assert kq.sensitivity(kq.hessian(X), np.array([1.0, 3.0]), "diag") == 30.0
    hb = np.array([[[1.0, 9.0], [9.0, 3.0]]])
    assert kq.sensitivity(kq.hessian(X), hb, "block") == 30.0
    # storage forms of one dense matrix keep the trace only when nothing is dropped from the diagonal
    rng = np.random.default_rng(18)
    H = spd(rng, 8)
    for form in ("diag", "block", "full"):
        assert np.isclose(kq.trace_form(kq.hg_forms(H, form, 4), form), np.trace(H), rtol=1e-14)
