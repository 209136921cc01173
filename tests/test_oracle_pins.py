"""Pins of the fp64 oracle against facts fixed outside it.

The pages print no worked numerical example of Muon or Newton-Schulz, so the
oracle is pinned by hand-derived examples (tests/golden/worked_examples.json),
closed forms on singular values, the polar factor from LAPACK's SVD,
equivariances, and the low-rank structure of MuonSSM's injections.  Each pin
is chosen so that a plausible slip in the oracle (a dropped or mis-signed
polynomial term, a wrong normalisation, EMA instead of heavy-ball momentum, a
missing Nesterov term, an ascent instead of a descent step, a transposed
operand) fails at least one of them; test_planted_mistakes_are_caught checks
that claim by planting those slips in copies of the oracle's steps.
"""
import json
import os

import numpy as np
import pytest

import oracle as orc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def p_scalar(x, a=1.5, b=-0.5, c=0.0):
    return a * x + b * x ** 3 + c * x ** 5


def spectral_expected(U, s, V, steps, coeffs, eps):
    """Closed form: NS_k(U diag(s) V^T) = U diag(p^k(s / (||s|| + eps))) V^T."""
    x = np.asarray(s, dtype=np.float64) / (np.linalg.norm(s) + eps)
    rows = coeffs if isinstance(coeffs[0], (tuple, list)) else [coeffs] * steps
    for r in rows[:steps]:
        x = p_scalar(x, *r)
    return (U * x) @ V.T


def haar(rng, n, k):
    q, r = np.linalg.qr(rng.standard_normal((n, k)))
    return q * np.sign(np.diag(r))


# ---------------------------------------------------------------------------
# Hand-derived examples
# ---------------------------------------------------------------------------
def test_worked_diag_example():
    g = GOLD["diag_3x2"]
    G = np.array(g["G"])
    X0, nu = orc.frobenius_normalize(G, 0.0)
    assert nu == g["nu"]
    np.testing.assert_allclose(np.diag(X0[:, :2]), g["X0_diag"], rtol=0, atol=1e-15)
    for k, key in ((1, "steps_1_diag"), (2, "steps_2_diag")):
        O, _ = orc.newton_schulz(G, k, eps=0.0)
        expect = np.zeros((2, 3))
        expect[0, 0], expect[1, 1] = g[key]
        np.testing.assert_allclose(O, expect, rtol=0, atol=1e-15)
        # the tall orientation gives the transpose
        Ot, _ = orc.newton_schulz(G.T, k, eps=0.0)
        np.testing.assert_allclose(Ot, expect.T, rtol=0, atol=1e-15)


def test_worked_momentum_example():
    g = GOLD["momentum_2x2"]
    M, G, beta = np.array(g["M"]), np.array(g["G"]), g["beta"]
    Mn = orc.momentum(M, G, beta)
    assert np.array_equal(Mn, np.array(g["M_new"]))
    assert np.array_equal(orc.update_direction(G, Mn, beta, True), np.array(g["U_nesterov"]))
    assert np.array_equal(orc.update_direction(G, Mn, beta, False), np.array(g["U_plain"]))
    out = orc.muon_step(np.zeros((2, 2)), M, G, beta=beta, lr=0.0, steps=0, eps=0.0)
    assert np.array_equal(out["M"], np.array(g["M_new"]))
    assert np.array_equal(out["U"], np.array(g["U_nesterov"]))


def test_worked_apply_example():
    g = GOLD["apply_rank1"]
    for steps in (0, 1, 5):
        out = orc.muon_step(np.array(g["W"]), np.zeros((2, 2)), np.array(g["G"]), beta=g["beta"],
                            lr=g["lr"], scale=g["scale"], steps=steps, eps=0.0)
        np.testing.assert_allclose(out["O"], np.array(g["O"]), rtol=0, atol=1e-15)
        np.testing.assert_allclose(out["W"], np.array(g["W_new"]), rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# Closed forms on singular values
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("m,n", [(24, 40), (40, 24), (16, 16)])
@pytest.mark.parametrize("steps", [1, 3, 5, 8])
def test_spectral_closed_form_cubic(m, n, steps):
    rng = np.random.default_rng(100 + m + n + steps)
    r = min(m, n)
    U, V = haar(rng, m, r), haar(rng, n, r)
    s = 10.0 ** (-3 * rng.random(r))
    G = (U * s) @ V.T
    O, nu = orc.newton_schulz(G, steps, eps=1e-7)
    assert abs(nu - np.linalg.norm(s)) < 1e-12 * nu
    np.testing.assert_allclose(O, spectral_expected(U, s, V, steps, (1.5, -0.5), 1e-7), atol=1e-12)


def test_spectral_closed_form_quintic_and_per_step():
    rng = np.random.default_rng(7)
    m, n = 20, 36
    U, V = haar(rng, m, m), haar(rng, n, m)
    s = rng.uniform(0.05, 1.0, m)
    G = (U * s) @ V.T
    quint = (3.4445, -4.7750, 2.0315)
    O, _ = orc.newton_schulz(G, 4, coeffs=quint, eps=0.0)
    np.testing.assert_allclose(O, spectral_expected(U, s, V, 4, quint, 0.0), atol=1e-12)
    per = [(1.5, -0.5, 0.0), (2.0, -1.5, 0.5), (1.2, -0.3, 0.1)]
    O, _ = orc.newton_schulz(G, 3, coeffs=np.array(per).ravel(), eps=0.0, per_step=True)
    np.testing.assert_allclose(O, spectral_expected(U, s, V, 3, per, 0.0), atol=1e-12)
    per2 = [(1.5, -0.5), (1.875, -1.25)]
    O, _ = orc.newton_schulz(G, 2, coeffs=np.array(per2).ravel(), eps=0.0, per_step=True)
    np.testing.assert_allclose(O, spectral_expected(U, s, V, 2, per2, 0.0), atol=1e-12)


def test_rank_one_fixed_point():
    rng = np.random.default_rng(3)
    u, v = rng.standard_normal(9), rng.standard_normal(14)
    G = 37.5 * np.outer(u, v)
    expect = np.outer(u, v) / (np.linalg.norm(u) * np.linalg.norm(v))
    for steps in (0, 1, 5, 12):
        O, _ = orc.newton_schulz(G, steps, eps=0.0)
        np.testing.assert_allclose(O, expect, atol=1e-14)


# ---------------------------------------------------------------------------
# Textbook routine: convergence to the polar factor
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("m,n", [(6, 10), (10, 6), (8, 8)])
def test_converges_to_polar_factor(m, n):
    rng = np.random.default_rng(11 * m + n)
    r = min(m, n)
    U, V = haar(rng, m, r), haar(rng, n, r)
    s = rng.uniform(1.0, 4.0, r)  # condition number <= 4
    G = (U * s) @ V.T
    O, _ = orc.newton_schulz(G, 30, eps=0.0)
    Us, _, Vt = np.linalg.svd(G, full_matrices=False)
    np.testing.assert_allclose(O, Us @ Vt, atol=1e-12)


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------
def test_normalisation_bounds():
    rng = np.random.default_rng(5)
    for shape in ((7, 30), (30, 7), (64, 128)):
        X = rng.standard_normal(shape) * 100
        X0, nu = orc.frobenius_normalize(X, 1e-7)
        assert abs(np.linalg.norm(X0) - nu / (nu + 1e-7)) < 1e-14
        assert np.linalg.svd(X0, compute_uv=False)[0] <= 1.0


def test_equivariances():
    rng = np.random.default_rng(9)
    m, n, k = 12, 20, 5
    G = rng.standard_normal((m, n))
    O, _ = orc.newton_schulz(G, k, eps=0.0)
    Q = haar(rng, m, m)
    Qr = haar(rng, n, n)
    np.testing.assert_allclose(orc.newton_schulz(Q @ G, k, eps=0.0)[0], Q @ O, atol=1e-13)
    np.testing.assert_allclose(orc.newton_schulz(G @ Qr, k, eps=0.0)[0], O @ Qr, atol=1e-13)
    np.testing.assert_allclose(orc.newton_schulz(G.T, k, eps=0.0)[0], O.T, atol=1e-14)
    np.testing.assert_allclose(orc.newton_schulz(-G, k, eps=0.0)[0], -O, atol=1e-14)
    np.testing.assert_allclose(orc.newton_schulz(3.7 * G, k, eps=0.0)[0], O, atol=1e-13)


def test_condition_number_does_not_grow():
    """'Muon Meets Mamba' (abstract): Muon lowers the condition number of the
    projection it trains.  For the cubic on [0, 1], p(y)/p(x) <= y/x when x <= y,
    so no Newton-Schulz step can raise sigma_max/sigma_min."""
    rng = np.random.default_rng(13)
    m, n = 16, 48
    U, V = haar(rng, m, m), haar(rng, n, m)
    s = 10.0 ** (-4 * rng.random(m))
    G = (U * s) @ V.T
    kappa = s.max() / s.min()
    prev = kappa
    for k in range(1, 9):
        sv = np.linalg.svd(orc.newton_schulz(G, k, eps=0.0)[0], compute_uv=False)
        assert sv[0] <= 1.0 + 1e-12
        cur = sv[0] / sv[-1]
        assert cur <= prev * (1 + 1e-9)
        prev = cur
    assert prev < kappa


def test_null_space_preserved():
    rng = np.random.default_rng(17)
    m, n, r = 10, 18, 4
    G = rng.standard_normal((m, r)) @ rng.standard_normal((r, n))
    _, _, Vt = np.linalg.svd(G)
    N = Vt[r:].T  # right null space
    O, _ = orc.newton_schulz(G, 5, eps=1e-7)
    assert np.abs(O @ N).max() < 1e-12
    assert np.abs(N.T @ O.T @ np.ones(m)).max() < 1e-12


def test_low_rank_injection_recurrence():
    """MuonSSM's injections are sums of value-key outer products ("MuonSSM",
    method section on momentum-augmented dynamics).  For X = V K^T every step
    stays of the form V C K^T with an r x r core:
    C0 = I / (nu + eps), nu^2 = tr((V^T V)(K^T K)),
    C <- a C + b C (K^T K) C^T (V^T V) C."""
    rng = np.random.default_rng(19)
    V, K = rng.standard_normal((64, 8)), rng.standard_normal((128, 8))
    X = V @ K.T
    VtV, KtK = V.T @ V, K.T @ K
    nu = np.sqrt(np.trace(VtV @ KtK))
    for steps in (1, 3, 5):
        C = np.eye(8) / (nu + 1e-7)
        for _ in range(steps):
            C = 1.5 * C - 0.5 * C @ KtK @ C.T @ VtV @ C
        O, nu_o = orc.newton_schulz(X, steps, eps=1e-7)
        assert abs(nu_o - nu) < 1e-10 * nu
        np.testing.assert_allclose(O, V @ C @ K.T, atol=1e-12)
    B = orc.ns_batched(np.stack([X, -2 * X, X.copy()]), 1)
    np.testing.assert_allclose(B[1], -B[0], atol=1e-14)


def test_zero_and_nan():
    O, nu = orc.newton_schulz(np.zeros((4, 6)), 5)
    assert nu == 0 and not O.any()
    W = np.ones((4, 6))
    out = orc.muon_step(W, np.zeros((4, 6)), np.zeros((4, 6)), beta=0.95, lr=0.02)
    assert np.array_equal(out["W"], W)
    G = np.ones((4, 6))
    G[1, 2] = np.nan
    assert np.isnan(orc.muon_step(W, np.zeros((4, 6)), G, beta=0.95, lr=0.02)["W"]).all()


def test_widening_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F80, 0x0001, 0x4049, 0x7F7F], np.uint16)
    vals = orc.widen_bf16(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[2] == 0.0
    assert np.signbit(vals[3]) and np.isinf(vals[4])
    assert vals[5] == 2.0 ** -133
    assert vals[6] == 3.140625
    assert vals[7] == (2 - 2 ** -7) * 2.0 ** 127


# ---------------------------------------------------------------------------
# Every planted slip must be caught by one of the pins above
# ---------------------------------------------------------------------------
def _ns_variant(U, steps, eps, slip):
    U = np.asarray(U, dtype=np.float64)
    tall = U.shape[0] > U.shape[1]
    X = U.T if tall else U
    nu = np.linalg.norm(X, 2) if slip == "spectral_norm" else np.sqrt(np.sum(X * X))
    X = X / (nu + eps)
    for _ in range(steps):
        A = X @ X.T
        if slip == "drop_b":
            X = 1.5 * X
        elif slip == "sign_b":
            X = 1.5 * X + 0.5 * (A @ X)
        elif slip == "transposed":
            # Gram taken on the wrong side; it only type-checks for square X
            X = 1.5 * X - 0.5 * ((X.T @ X) @ X)
        else:
            X = 1.5 * X - 0.5 * (A @ X)
    return X.T if tall else X


@pytest.mark.parametrize("slip", ["drop_b", "sign_b", "spectral_norm", "transposed"])
def test_planted_mistakes_are_caught(slip):
    g = GOLD["diag_3x2"]
    G = np.array(g["G"])
    expect = np.zeros((2, 3))
    expect[0, 0], expect[1, 1] = g["steps_1_diag"]
    assert np.allclose(_ns_variant(G, 1, 0.0, None), expect, atol=1e-15)
    caught = False
    if slip != "transposed":  # the wrong-side Gram does not type-check on a 2 x 3 matrix
        caught = not np.allclose(_ns_variant(G, 1, 0.0, slip), expect, atol=1e-12)
    rng = np.random.default_rng(1)
    U, V = haar(rng, 9, 9), haar(rng, 9, 9)
    s = rng.uniform(0.1, 1.0, 9)
    Gs = (U * s) @ V.T  # square and not normal
    closed = spectral_expected(U, s, V, 3, (1.5, -0.5), 0.0)
    assert np.allclose(_ns_variant(Gs, 3, 0.0, None), closed, atol=1e-12)
    caught = caught or not np.allclose(_ns_variant(Gs, 3, 0.0, slip), closed, atol=1e-12)
    assert caught


def test_planted_momentum_slips_are_caught():
    g = GOLD["momentum_2x2"]
    M, G, beta = np.array(g["M"]), np.array(g["G"]), g["beta"]
    ema = beta * M + (1 - beta) * G
    assert not np.array_equal(ema, np.array(g["M_new"]))
    no_nesterov = ema
    assert not np.array_equal(no_nesterov, np.array(g["U_nesterov"]))
    a = GOLD["apply_rank1"]
    ascent = np.array(a["W"]) + a["lr"] * a["scale"] * np.array(a["O"])
    assert not np.allclose(ascent, np.array(a["W_new"]))


# ---------------------------------------------------------------------------
# The GPU path may run the iteration in accumulated form: every iterate is
# Q X0 with Q a polynomial in A_0 = X0 X0^T, so A_k = X_k X_k^T obeys
# A_{k+1} = A_k B_k^2 with B_k = a_k I + b_k A_k, and O = B_{n-1} ... B_0 X0.
# That is an identity of the iteration the oracle runs; it is pinned in fp64
# here so that the GPU's choice of schedule is a question of rounding only.
# ---------------------------------------------------------------------------
def _accumulated(U, steps, rows):
    tall = U.shape[0] > U.shape[1]
    X0 = U.T if tall else U
    X0 = X0 / np.linalg.norm(X0)
    A = X0 @ X0.T
    Q = np.eye(A.shape[0])
    for k in range(steps):
        a, b = rows[k]
        B = a * np.eye(A.shape[0]) + b * A
        Q = B @ Q
        A = A @ B @ B
    O = Q @ X0
    return O.T if tall else O


@pytest.mark.parametrize("m,n,steps", [(6, 15, 2), (12, 40, 5), (30, 9, 8), (16, 16, 3)])
def test_accumulated_schedule_is_the_iteration(m, n, steps):
    rng = np.random.default_rng(m * 100 + n)
    U = rng.standard_normal((m, n)) * np.exp(rng.uniform(-3, 0, (m, 1)))
    ref, _ = orc.newton_schulz(U, steps, eps=0.0)
    assert np.allclose(_accumulated(U, steps, [(1.5, -0.5)] * steps), ref, rtol=0, atol=1e-12)
    rows = [(2.0 - 0.1 * k, -0.6 + 0.02 * k) for k in range(steps)]
    ref2, _ = orc.newton_schulz(U, steps, coeffs=rows, eps=0.0, per_step=True)
    assert np.allclose(_accumulated(U, steps, rows), ref2, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Factored injections X = V K^T ("MuonSSM", method section on the low-rank
# value-key injections): the oracle's core C must reproduce the dense result
# and agree with two independent routes to it.
# ---------------------------------------------------------------------------
def _core_recurrence(V, K, steps, rows, eps):
    P, S = V.T @ V, K.T @ K
    nu = np.sqrt(np.trace(P @ S))
    C = np.eye(V.shape[1]) / (nu + eps)
    for a, b, c in rows:
        N = C @ S @ C.T @ P
        C = a * C + b * N @ C + c * N @ N @ C
    return C


@pytest.mark.parametrize("m,n,r,steps", [(64, 128, 8, 1), (64, 128, 8, 5), (32, 96, 4, 3), (128, 64, 8, 2),
                                         (40, 40, 1, 4)])
def test_factored_ns_core(m, n, r, steps):
    rng = np.random.default_rng(m + n + r + steps)
    V, K = rng.standard_normal((m, r)), rng.standard_normal((n, r))
    O, C, nu = orc.factored_ns(V, K, steps)
    np.testing.assert_allclose(V @ C @ K.T, O, rtol=0, atol=1e-12)  # the core reproduces the dense result
    np.testing.assert_allclose(C, _core_recurrence(V, K, steps, [(1.5, -0.5, 0.0)] * steps, 1e-7), rtol=1e-10,
                               atol=1e-12)
    rows = [(2.0, -1.5, 0.5)] * steps
    O5, C5, _ = orc.factored_ns(V, K, steps, coeffs=rows, per_step=True)
    np.testing.assert_allclose(C5, _core_recurrence(V, K, steps, rows, 1e-7), rtol=1e-9, atol=1e-12)


def test_factored_ns_orthonormal_closed_form():
    """V = Qv diag(alpha), K = Qk with orthonormal columns: X has singular
    values alpha, so C_ii = p^k(alpha_i / (||alpha|| + eps)) / alpha_i."""
    rng = np.random.default_rng(7)
    Qv, _ = np.linalg.qr(rng.standard_normal((64, 6)))
    Qk, _ = np.linalg.qr(rng.standard_normal((128, 6)))
    alpha = np.array([3.0, 1.0, 0.5, 0.25, 0.1, 0.01])
    for steps in (1, 3, 6):
        O, C, nu = orc.factored_ns(Qv * alpha, Qk, steps)
        x = alpha / (np.linalg.norm(alpha) + 1e-7)
        for _ in range(steps):
            x = 1.5 * x - 0.5 * x ** 3
        np.testing.assert_allclose(C, np.diag(x / alpha), rtol=0, atol=1e-12)
        assert abs(nu - np.linalg.norm(alpha)) < 1e-12


# ---------------------------------------------------------------------------
# Spectral cap ("An Isotropy-Preserving Spectral Cap for Muon"): pins of the
# reading that the capped update removes exactly the first-order growth of the
# top singular value and nothing else.
# ---------------------------------------------------------------------------
def _gapped(rng, m, n, top=5.0):
    Uq, _ = np.linalg.qr(rng.standard_normal((m, min(m, n))))
    Vq, _ = np.linalg.qr(rng.standard_normal((n, min(m, n))))
    s = np.concatenate([[top], rng.uniform(0.1, 1.0, min(m, n) - 1)])
    return (Uq * s) @ Vq.T, Uq[:, 0], Vq[:, 0], top


def test_cap_removes_first_order_growth():
    rng = np.random.default_rng(41)
    W, u1, v1, s1 = _gapped(rng, 40, 70)
    O = rng.standard_normal((40, 70))
    O -= (abs(u1 @ O @ v1) + 0.5) * np.outer(u1, v1)    # make u1^T O v1 < 0: W - eps O grows sigma_1
    c = u1 @ O @ v1
    O2, gamma = orc.spectral_cap_update(O, u1, v1, s1, cap=1.0)
    assert gamma == c and abs(u1 @ O2 @ v1) < 1e-12
    # the rest of O is untouched: O - O2 is rank one along u1 v1^T
    np.testing.assert_allclose(O - O2, c * np.outer(u1, v1), atol=1e-12)
    for h in (1e-3, 1e-4):
        grow = np.linalg.svd(W - h * O, compute_uv=False)[0] - s1
        capped = np.linalg.svd(W - h * O2, compute_uv=False)[0] - s1
        assert abs(grow + h * c) < 50 * h * h          # first order: -h u^T O v > 0
        assert abs(capped) < 50 * h * h                # removed: second order only


def test_cap_inactive_cases():
    rng = np.random.default_rng(42)
    W, u1, v1, s1 = _gapped(rng, 30, 20)
    O = rng.standard_normal((30, 20))
    O += (abs(u1 @ O @ v1) + 0.5) * np.outer(u1, v1)    # u1^T O v1 > 0: sigma_1 shrinks
    O2, gamma = orc.spectral_cap_update(O, u1, v1, s1, cap=0.0)
    assert gamma == 0.0 and np.array_equal(O2, O)
    O3 = O - 2 * (u1 @ O @ v1) * np.outer(u1, v1)       # now it would grow, but sigma is below the cap
    O4, gamma = orc.spectral_cap_update(O3, u1, v1, s1, cap=s1 + 1.0)
    assert gamma == 0.0 and np.array_equal(O4, O3)


def test_power_step_converges_to_lapack_pair():
    rng = np.random.default_rng(43)
    W, u1, v1, s1 = _gapped(rng, 50, 80, top=3.0)
    u, v = rng.standard_normal(50), rng.standard_normal(80)
    u, v = u / np.linalg.norm(u), v / np.linalg.norm(v)
    for _ in range(60):
        u, v, sig = orc.power_step(W, u, v)
    assert abs(abs(u @ u1) - 1) < 1e-10 and abs(abs(v @ v1) - 1) < 1e-10
    assert abs(sig - s1) < 1e-9
    # rank one: exact after one step from any start not orthogonal to it
    a, b = rng.standard_normal(12), rng.standard_normal(9)
    u, v, sig = orc.power_step(2.5 * np.outer(a, b), rng.standard_normal(12), rng.standard_normal(9))
    np.testing.assert_allclose(np.abs(u), np.abs(a) / np.linalg.norm(a), atol=1e-14)
    np.testing.assert_allclose(np.abs(v), np.abs(b) / np.linalg.norm(b), atol=1e-14)
    # zero weight: the vectors stay
    u0, v0 = rng.standard_normal(12), rng.standard_normal(9)
    u, v, sig = orc.power_step(np.zeros((12, 9)), u0, v0)
    assert sig == 0.0 and np.array_equal(u, u0) and np.array_equal(v, v0)


def test_capped_step_matches_uncapped_when_off():
    rng = np.random.default_rng(44)
    W, M, G = rng.standard_normal((24, 40)), rng.standard_normal((24, 40)), rng.standard_normal((24, 40))
    u, v = rng.standard_normal(24), rng.standard_normal(40)
    u, v = u / np.linalg.norm(u), v / np.linalg.norm(v)
    ref = orc.muon_step(W, M, G, beta=0.95, lr=0.02, steps=3)
    out = orc.muon_step_capped(W, M, G, u, v, 0.0, cap=1e30, beta=0.95, lr=0.02, steps=3)
    assert out["gamma"] == 0.0
    np.testing.assert_array_equal(out["W"], ref["W"])
    np.testing.assert_array_equal(out["O"], ref["O"])


# ---------------------------------------------------------------------------
# Companion AdamW: closed forms of the bias-corrected moments.
# ---------------------------------------------------------------------------
def test_adamw_first_step_and_constant_gradient():
    rng = np.random.default_rng(51)
    p, g = rng.standard_normal(1000), rng.standard_normal(1000)
    kw = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    # step 1 from zero moments: m_hat = g, v_hat = g^2
    p1, m1, v1 = orc.adamw_step(p, g, np.zeros(1000), np.zeros(1000), step=1, **kw)
    np.testing.assert_allclose(m1, 0.1 * g, rtol=1e-14)
    np.testing.assert_allclose(v1, 0.05 * g * g, rtol=1e-14)  # 1 - 0.95 is not exact in binary
    np.testing.assert_allclose(p1, p * (1 - 1e-4) - 1e-3 * g / (np.abs(g) + 1e-8), rtol=1e-12, atol=1e-15)
    # a constant gradient keeps m_hat = g and v_hat = g^2 at every step
    pk, mk, vk = p, np.zeros(1000), np.zeros(1000)
    for t in range(1, 30):
        prev = pk
        pk, mk, vk = orc.adamw_step(pk, g, mk, vk, step=t, **kw)
        np.testing.assert_allclose(pk, prev * (1 - 1e-4) - 1e-3 * g / (np.abs(g) + 1e-8), rtol=1e-11, atol=1e-14)


def test_adamw_hand_example_and_zero_gradient():
    # one scalar by hand: p=1, g=2, m=0.5, v=1, b1=0.5, b2=0.75, step 2, lr 0.1, wd 0.5, eps 0
    p2, m2, v2 = orc.adamw_step(np.array([1.0]), np.array([2.0]), np.array([0.5]), np.array([1.0]), lr=0.1,
                                beta1=0.5, beta2=0.75, eps=0.0, weight_decay=0.5, step=2)
    # m' = 0.25 + 1 = 1.25, v' = 0.75 + 0.25*4 = 1.75, m_hat = 1.25/0.75, v_hat = 1.75/0.4375 = 4
    assert m2[0] == 1.25 and v2[0] == 1.75
    assert abs(p2[0] - (0.95 - 0.1 * (1.25 / 0.75) / 2.0)) < 1e-15
    # zero gradient: only the moments decay and the weight decays
    p3, m3, v3 = orc.adamw_step(np.array([3.0]), np.array([0.0]), np.array([0.0]), np.array([0.0]), lr=0.01,
                                beta1=0.9, beta2=0.99, eps=1e-8, weight_decay=0.2, step=5)
    assert m3[0] == 0.0 and v3[0] == 0.0 and abs(p3[0] - 3.0 * (1 - 0.002)) < 1e-15


# ---- spectral diagnostics ----------------------------------------------------
def haar(rng, n, k):
    q, r = np.linalg.qr(rng.standard_normal((n, k)))
    return q * np.sign(np.diag(r))


def test_lanczos_start_hand_values():
    # (i * 2654435769) mod 2^32 for i = 0..3, by hand: 0, 2654435769,
    # 5308871538 - 2^32 = 1013904242, 7963307307 - 2^32 = 3668340011; top 24
    # bits: 0, 10368889, 3960563, 14329453
    want = np.array([0, 10368889, 3960563, 14329453]) / 2.0 ** 24 - 0.5
    assert np.array_equal(orc.lanczos_start(4), want)
    q = orc.lanczos_start(1000)
    assert abs(q.mean()) < 2e-3 and q.min() >= -0.5 and q.max() < 0.5  # equidistributed


def test_orth_error_closed_form_both_orientations():
    rng = np.random.default_rng(31)
    for m, n in ((40, 90), (90, 40)):
        s = min(m, n)
        sig = rng.uniform(0.1, 1.7, s)
        A = haar(rng, m, s) @ np.diag(sig) @ haar(rng, n, s).T
        want = np.sqrt(np.sum((sig ** 2 - 1.0) ** 2) / s)
        d = orc.spectral_diagnostics(A, s)
        assert abs(d["orth_err"] - want) <= 1e-12 * want
        # iters = s: the Krylov space is everything, Ritz extremes = singular extremes
        assert abs(d["sigma_max"] - sig.max()) <= 1e-10 and abs(d["sigma_min"] - sig.min()) <= 1e-10


def test_lanczos_full_run_matches_lapack_svd():
    rng = np.random.default_rng(5)
    A = rng.standard_normal((60, 150))
    sv = np.linalg.svd(A, compute_uv=False)
    lo, hi = orc.lanczos_extremes(A @ A.T, 60)
    assert abs(hi - sv[0] ** 2) <= 1e-10 * sv[0] ** 2 and abs(lo - sv[-1] ** 2) <= 1e-10 * sv[0] ** 2


def test_lanczos_ritz_bounds_and_monotone():
    """Ritz values interlace: the extreme ones lie inside the spectrum and move
    outwards as the Krylov space grows."""
    rng = np.random.default_rng(6)
    s = 80
    lam = np.sort(rng.uniform(0.05, 2.0, s))
    Qm = haar(rng, s, s)
    H = Qm @ np.diag(lam) @ Qm.T
    prev_lo, prev_hi = np.inf, -np.inf
    for k in (1, 2, 4, 8, 16, 32, 80):
        lo, hi = orc.lanczos_extremes(H, k)
        assert lam[0] - 1e-12 <= lo <= hi <= lam[-1] + 1e-12
        assert lo <= prev_lo + 1e-12 and hi >= prev_hi - 1e-12
        prev_lo, prev_hi = lo, hi
    assert abs(prev_lo - lam[0]) < 1e-10 and abs(prev_hi - lam[-1]) < 1e-10


def test_lanczos_two_distinct_eigenvalues_exact_after_two_steps():
    rng = np.random.default_rng(8)
    s = 12
    Qm = haar(rng, s, s)
    lam = np.array([4.0] * 5 + [0.25] * 7)
    H = Qm @ np.diag(lam) @ Qm.T
    lo, hi = orc.lanczos_extremes(H, 2)
    assert abs(lo - 0.25) < 1e-12 and abs(hi - 4.0) < 1e-12
    # the Krylov space is invariant after two steps: the run stops there
    lo, hi = orc.lanczos_extremes(H, 12)
    assert abs(lo - 0.25) < 1e-12 and abs(hi - 4.0) < 1e-12
    # a multiple of the identity: one step
    lo, hi = orc.lanczos_extremes(3.0 * np.eye(9), 9)
    assert abs(lo - 3.0) < 1e-14 and abs(hi - 3.0) < 1e-14


def test_lanczos_2x2_closed_form_and_degenerate_inputs():
    A = np.array([[1.0, 2.0, 0.5], [-1.0, 0.25, 3.0]])
    H = A @ A.T
    a, b, c = H[0, 0], H[0, 1], H[1, 1]
    r = np.sqrt(((a - c) / 2) ** 2 + b * b)
    lo, hi = orc.lanczos_extremes(H, 2)
    assert abs(lo - ((a + c) / 2 - r)) < 1e-12 and abs(hi - ((a + c) / 2 + r)) < 1e-12
    z = orc.spectral_diagnostics(np.zeros((5, 9)), 5)
    assert z["orth_err"] == 1.0 and z["sigma_max"] == 0.0 and z["sigma_min"] == 0.0
    eye = orc.spectral_diagnostics(np.hstack([np.eye(6), np.zeros((6, 3))]), 6)
    assert eye["orth_err"] == 0.0 and abs(eye["sigma_max"] - 1) < 1e-15 and abs(eye["sigma_min"] - 1) < 1e-15
    bad = np.ones((4, 7))
    bad[1, 2] = np.nan
    d = orc.spectral_diagnostics(bad, 4)
    assert np.isnan(d["orth_err"]) and np.isnan(d["sigma_max"]) and np.isnan(d["sigma_min"])


# ---------------------------------------------------------------------------
# Batched Newton-Schulz and the capped step's outputs, pinned independently of
# the oracle's own code paths.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("m,n", [(6, 10), (10, 6)])
@pytest.mark.parametrize("steps", [0, 1, 5])
def test_ns_batched_closed_form_per_matrix(m, n, steps):
    """Every matrix of the stack is normalised by its own Frobenius norm and
    iterated the given number of steps: built as U_i diag(s_i) V_i^T with
    scales that differ by orders of magnitude, each must equal the singular
    value closed form of its own factors (a wrong step count, a norm taken
    over the whole stack or coefficients not passed through all fail)."""
    rng = np.random.default_rng(300 + steps)
    k = min(m, n)
    mats, want = [], []
    for i, scale in enumerate((1e-3, 1.0, 40.0, 0.5)):
        U, V = haar(rng, m, k), haar(rng, n, k)
        s = scale * rng.uniform(0.05, 1.0, k)
        mats.append((U * s) @ V.T)
        want.append(spectral_expected(U, s, V, steps, (1.5, -0.5), 1e-7))
    out = orc.ns_batched(np.stack(mats), steps)
    for i in range(len(mats)):
        np.testing.assert_allclose(out[i], want[i], atol=1e-12)
    # per-step coefficients reach every matrix of the stack
    rows = [(3.4445, -4.7750, 2.0315)] * steps
    if steps:
        outq = orc.ns_batched(np.stack(mats), steps, coeffs=[c for r in rows for c in r], per_step=True)
        for i, M in enumerate(mats):
            Uu, s, Vt = np.linalg.svd(M, full_matrices=False)
            np.testing.assert_allclose(outq[i], spectral_expected(Uu, s, Vt.T, steps, rows, 1e-7), atol=1e-11)


def test_capped_step_active_increment_and_tracked_pair():
    """Cap active: with W built from its SVD and (u, v) = W's exact top pair,
    a gradient dominated by -u v^T makes u^T O v < 0.  The weight increment
    must be -lr (O - gamma u v^T) with O the singular-value closed form of
    the direction U = (1 + beta) G (M = 0) and gamma = u^T O v; the tracked
    triple must come from one power step on the new weight, started from the
    old (u, v): computed here from W' through its own SVD factors, and
    different from the same step taken on the old weight."""
    rng = np.random.default_rng(310)
    m, n, beta, lr, steps = 24, 40, 0.95, 0.02, 5
    Uw, Vw = haar(rng, m, m), haar(rng, n, m)
    sw = np.concatenate([[3.0], rng.uniform(0.2, 1.0, m - 1)])
    W = (Uw * sw) @ Vw.T
    u, v, sigma = Uw[:, 0], Vw[:, 0], 3.0
    G = -5.0 * np.outer(u, v) + 0.1 * rng.standard_normal((m, n))
    out = orc.muon_step_capped(W, np.zeros((m, n)), G, u, v, sigma, cap=2.0, beta=beta, lr=lr, steps=steps)
    Ug, sg, Vgt = np.linalg.svd((1 + beta) * G, full_matrices=False)
    O_cf = spectral_expected(Ug, sg, Vgt.T, steps, (1.5, -0.5), 1e-7)
    c = float(u @ O_cf @ v)
    assert c < 0 and abs(out["gamma"] - c) < 1e-12
    np.testing.assert_allclose(out["O_uncapped"], O_cf, atol=1e-12)
    np.testing.assert_allclose(out["W"] - W, -lr * (O_cf - c * np.outer(u, v)), atol=1e-13)
    assert abs(u @ out["O"] @ v) < 1e-12
    # the new triple: W' v / ||W' v|| etc. through the SVD factors of W'
    Up, sp, Vpt = np.linalg.svd(out["W"], full_matrices=False)
    y = Up @ (sp * (Vpt @ v))
    z = Vpt.T @ (sp * (Up.T @ u))
    np.testing.assert_allclose(out["u"], y / np.linalg.norm(y), atol=1e-12)
    np.testing.assert_allclose(out["v"], z / np.linalg.norm(z), atol=1e-12)
    assert abs(out["sigma"] - np.linalg.norm(y)) < 1e-12
    u_old, v_old, s_old = orc.power_step(W, u, v)
    assert np.abs(out["u"] - u_old).max() > 1e-6 or abs(out["sigma"] - s_old) > 1e-6
    # cap not reached (sigma below it): the update is the plain one
    off = orc.muon_step_capped(W, np.zeros((m, n)), G, u, v, sigma, cap=3.5, beta=beta, lr=lr, steps=steps)
    assert off["gamma"] == 0.0
    np.testing.assert_allclose(off["W"] - W, -lr * O_cf, atol=1e-13)


@pytest.mark.parametrize("k", [2, 3, 5])
def test_lanczos_ritz_values_are_the_krylov_projection(k):
    """For k < s the Lanczos estimates are the extreme eigenvalues of H
    projected onto the Krylov space span{q, Hq, ..., H^(k-1) q} of the start
    vector (Rayleigh-Ritz): here that space is orthonormalised by a QR of the
    Krylov matrix itself, not by the Lanczos recurrence."""
    rng = np.random.default_rng(320 + k)
    s = 40
    lam = np.sort(rng.uniform(0.1, 2.0, s))
    Qm = haar(rng, s, s)
    H = Qm @ np.diag(lam) @ Qm.T
    q = orc.lanczos_start(s)
    K = np.empty((s, k))
    K[:, 0] = q / np.linalg.norm(q)
    for j in range(1, k):
        w = H @ K[:, j - 1]
        K[:, j] = w / np.linalg.norm(w)
    B, _ = np.linalg.qr(K)
    ev = np.linalg.eigvalsh(B.T @ H @ B)
    lo, hi = orc.lanczos_extremes(H, k)
    assert abs(lo - ev[0]) < 1e-10 and abs(hi - ev[-1]) < 1e-10


# ---------------------------------------------------------------------------
# Momentum pathway of MuonSSM (momentum-augmented state update): M_t and S_t
# ---------------------------------------------------------------------------
def test_momentum_recurrence_three_tokens_written_out():
    """Three tokens expanded by hand from M_t = b M_{t-1} + U_t and
    S_t = a_t S_{t-1} + M_t:
      M_3 = b^3 M0 + b^2 U1 + b U2 + U3
      S_3 = a3 a2 a1 S0 + (a3 a2 b + a3 b^2 + b^3) M0 + (a3 a2 + a3 b + b^2) U1
            + (a3 + b) U2 + U3
    An off-by-one in either recurrence (S fed M_{t-1}, M fed before S, the
    decay applied to M) changes these coefficients."""
    rng = np.random.default_rng(71)
    M0, S0 = rng.standard_normal((2, 3, 5))
    U1, U2, U3 = rng.standard_normal((3, 3, 5))
    a1, a2, a3 = 0.91, 0.63, 0.77
    b = 0.85
    M, S = orc.momentum_recurrence([U1, U2, U3], [a1, a2, a3], b, M0, S0)
    M_ref = b ** 3 * M0 + b ** 2 * U1 + b * U2 + U3
    S_ref = (a3 * a2 * a1 * S0 + (a3 * a2 * b + a3 * b ** 2 + b ** 3) * M0 + (a3 * a2 + a3 * b + b ** 2) * U1
             + (a3 + b) * U2 + U3)
    np.testing.assert_allclose(M, M_ref, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(S, S_ref, rtol=1e-14, atol=1e-14)
    M_only, S_none = orc.momentum_recurrence([U1, U2, U3], None, b, M0)
    assert S_none is None
    np.testing.assert_allclose(M_only, M_ref, rtol=1e-14, atol=1e-14)


def test_momentum_recurrence_is_block_affine_in_any_bracketing():
    """The pages state that the memory and momentum states together follow a
    block-affine recurrence, so a parallel scan may compose the per-token maps
    in any bracketing.  Each token is the map (S, M) -> (a S + b M + U,
    b M + U); composing them as a balanced tree of (2 x 2 coefficient matrix,
    offset pair) maps must give the sequential result."""
    rng = np.random.default_rng(72)
    T, b = 13, 0.9
    U = rng.standard_normal((T, 4, 6))
    a = rng.uniform(0.5, 1.0, T)
    M0, S0 = rng.standard_normal((2, 4, 6))

    def token_map(t):
        return np.array([[a[t], b], [0.0, b]]), (U[t], U[t])

    def compose(f, g):  # g after f
        Af, (bs_f, bm_f) = f
        Ag, (bs_g, bm_g) = g
        return Ag @ Af, (Ag[0, 0] * bs_f + Ag[0, 1] * bm_f + bs_g, Ag[1, 0] * bs_f + Ag[1, 1] * bm_f + bm_g)

    def tree(lo, hi):
        if hi - lo == 1:
            return token_map(lo)
        mid = (lo + hi) // 2
        return compose(tree(lo, mid), tree(mid, hi))

    A, (bs, bm) = tree(0, T)
    S_scan = A[0, 0] * S0 + A[0, 1] * M0 + bs
    M_scan = A[1, 0] * S0 + A[1, 1] * M0 + bm
    M, S = orc.momentum_recurrence(U, a, b, M0, S0)
    np.testing.assert_allclose(M, M_scan, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, S_scan, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("steps", [1, 5])
def test_ssm_momentum_rank_one_closed_form(steps):
    """Rank-1 injections X_t = v_t k_t^T have one singular value, so the
    Frobenius-normalised matrix has sigma = 1 (up to eps), a fixed point of
    the cubic (1.5 - 0.5 = 1): U_t = v_t k_t^T / (|v_t| |k_t|).  The final
    states are then weighted sums with weights written as explicit products
    and sums (no recurrence):
      M_T = b^T M0 + sum_u b^(T-u) U_u
      S_T = (prod_t a_t) S0 + sum_t g_t b^t M0 + sum_u (sum_{t>=u} g_t b^(t-u)) U_u,
    g_t = prod_{s>t} a_s (tokens numbered 1..T)."""
    rng = np.random.default_rng(73)
    T, m, n, b = 6, 5, 7, 0.8
    V = rng.standard_normal((T, m, 1))
    K = rng.standard_normal((T, n, 1))
    a = rng.uniform(0.6, 1.0, T)
    M0, S0 = rng.standard_normal((2, m, n))
    Uc = [np.outer(V[t, :, 0], K[t, :, 0]) / (np.linalg.norm(V[t]) * np.linalg.norm(K[t])) for t in range(T)]
    g = [np.prod(a[t + 1:]) for t in range(T)]  # token t + 1 in 1-based numbering
    M_ref = b ** T * M0 + sum(b ** (T - 1 - u) * Uc[u] for u in range(T))
    S_ref = (np.prod(a) * S0 + sum(g[t] * b ** (t + 1) for t in range(T)) * M0
             + sum(sum(g[t] * b ** (t - u) for t in range(u, T)) * Uc[u] for u in range(T)))
    M, S = orc.ssm_momentum(V, K, a, b, M0, S0, steps=steps, eps=0.0)
    np.testing.assert_allclose(M, M_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-12)


def test_ssm_momentum_single_token_is_the_ns_step():
    """With b = 0 and a = 0 both states equal the newest token's Newton-Schulz
    result, whatever M0 and S0 held."""
    rng = np.random.default_rng(74)
    V = rng.standard_normal((3, 16, 8))
    K = rng.standard_normal((3, 24, 8))
    M0, S0 = rng.standard_normal((2, 16, 24))
    M, S = orc.ssm_momentum(V, K, np.zeros(3), 0.0, M0, S0, steps=1)
    O, _ = orc.newton_schulz(V[2] @ K[2].T, 1)
    np.testing.assert_allclose(M, O, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S, O, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("slip", ["s_uses_old_m", "decay_on_m", "ema_momentum", "s_skips_momentum"])
def test_planted_recurrence_slips_are_caught(slip):
    """Plausible misreadings of the momentum pathway, planted in a copy of the
    recurrence, each break the written-out three-token pin."""
    rng = np.random.default_rng(75)
    M0, S0 = rng.standard_normal((2, 3, 4))
    U = rng.standard_normal((3, 3, 4))
    a, b = [0.91, 0.63, 0.77], 0.85

    def slipped():
        M, S = M0.copy(), S0.copy()
        for t in range(3):
            M_old = M
            if slip == "decay_on_m":
                M = a[t] * M + U[t]
            elif slip == "ema_momentum":
                M = b * M + (1 - b) * U[t]
            else:
                M = b * M + U[t]
            if slip == "s_uses_old_m":
                S = a[t] * S + M_old
            elif slip == "s_skips_momentum":
                S = a[t] * S + U[t]
            else:
                S = a[t] * S + M
        return M, S

    M_ref, S_ref = orc.momentum_recurrence(U, a, b, M0, S0)
    M, S = slipped()
    assert not (np.allclose(M, M_ref, rtol=1e-6) and np.allclose(S, S_ref, rtol=1e-6))
