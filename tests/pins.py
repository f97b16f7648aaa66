"""Pins: checks of the CPU oracle against facts fixed by the pages and by mathematics.

None of these re-types the oracle's matrix iteration. They use:

* the scalar form of the quintic map, p(s) = a s + b s^3 + c s^5, which the iteration of
  page "深入解析KellerJordan/modded-nanogpt中的训练架构与优化技术" (section
  "Newton-Schulz正交化") reduces to on each singular value, evaluated in exact rational
  arithmetic or as a scalar polynomial;
* numpy's SVD / symmetric eigensolver as independent routes to the same matrix function;
* the closed form of SGD/Nesterov momentum with constant coefficients (section "核心算法"
  of the same page names standard SGD momentum and nesterov=True);
* invariances of an odd matrix polynomial (sign, positive scale, orthogonal factors,
  transposition, zero padding).

Each pin is a function that raises AssertionError when the oracle disagrees. They look up
the oracle's functions through the module at call time, so a test can plant a mistake in
the oracle (monkeypatch) and check that some pin catches it.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

import oracle.muon as om

A_, B_, C_ = 3.4445, -4.7750, 2.0315
FA, FB, FC = Fraction("3.4445"), Fraction("-4.7750"), Fraction("2.0315")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ns_quintic_hand_expansion.txt")


def p_frac(s: Fraction) -> Fraction:
    return FA * s + FB * s ** 3 + FC * s ** 5


def p_float(s):
    s = np.asarray(s, dtype=np.float64)
    return A_ * s + B_ * s ** 3 + C_ * s ** 5


def p_iter(s, k: int):
    for _ in range(k):
        s = p_float(s)
    return s


def _rng(seed):
    return np.random.default_rng(seed)


def _rel(x, y):
    return float(np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300))


def _ns_normalised(G, steps=5, eps=0.0, literal=False):
    O, _ = om.orthogonalize(np.asarray(G, np.float64), steps, om.DEFAULT_ABC, eps, literal)
    return O


# ---------------------------------------------------------------------------------------
def pin_p1_hand_expansion():
    """P1: one round on diagonal inputs equals the hand-expanded polynomial (golden file)."""
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        s, val, rounds = line.split()
        rows.append((Fraction(s), Fraction(val), int(rounds)))
    for s, val, rounds in rows:
        if rounds == 1:
            assert p_frac(s) == val, (s, p_frac(s), val)          # the fixture's arithmetic
            X = np.diag([float(s), 0.5])
            out = om.newton_schulz(X, 1)
            assert abs(out[0, 0] - float(val)) < 1e-14, (s, out[0, 0], val)
            assert abs(out[1, 0]) < 1e-15 and abs(out[0, 1]) < 1e-15
    assert om.DEFAULT_ABC == (A_, B_, C_)


def pin_p2_diagonal_worked_example():
    """P2: G = diag(3, 4) -> Frobenius 5 -> diag(0.6, 0.8) -> five rounds (golden file)."""
    G = np.diag([3.0, 4.0])
    O = _ns_normalised(G, 5, eps=0.0)
    s, t = Fraction(3, 5), Fraction(4, 5)
    for _ in range(5):
        s, t = p_frac(s), p_frac(t)
    want = np.diag([float(s), float(t)])
    assert np.max(np.abs(O - want)) < 1e-13, (O, want)
    gold = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    g5 = {Fraction(r[0]): float(r[1]) for r in gold if r[2] == "5"}
    assert abs(O[0, 0] - g5[Fraction(3, 5)]) < 1e-11 and abs(O[1, 1] - g5[Fraction(4, 5)]) < 1e-11


def pin_p3_symmetric_2x2():
    """P3: [[2,1],[1,2]] has eigenvectors (1,1)/sqrt2, (1,-1)/sqrt2 and eigenvalues 3, 1; the
    result is Q diag(p^5(3/sqrt10), p^5(1/sqrt10)) Q^T, which is not the polar factor I."""
    G = np.array([[2.0, 1.0], [1.0, 2.0]])
    O = _ns_normalised(G, 5, eps=0.0)
    p1, p2 = p_iter(3 / np.sqrt(10), 5), p_iter(1 / np.sqrt(10), 5)
    want = np.array([[(p1 + p2) / 2, (p1 - p2) / 2], [(p1 - p2) / 2, (p1 + p2) / 2]])
    assert np.max(np.abs(O - want)) < 1e-13, (O, want)
    assert np.max(np.abs(O - np.eye(2))) > 0.05


def pin_p4_svd_identity():
    """P4: NS5(G/||G||_F) = U diag(p^5(sigma_i/||G||_F)) V^T on random inputs."""
    for k, (m, n) in enumerate([(2, 2), (4, 6), (8, 8), (64, 256), (96, 32), (5, 3)]):
        G = _rng(100 + k).standard_normal((m, n))
        O = _ns_normalised(G, 5, eps=0.0)
        U, S, Vt = np.linalg.svd(G, full_matrices=False)
        want = (U * p_iter(S / np.linalg.norm(G), 5)) @ Vt
        assert _rel(O, want) < 1e-11, ((m, n), _rel(O, want))


def pin_p5_band():
    """P5: output singular values lie in the band [p(s2), p(s1)] where s1 < s2 are the
    critical points of p (p'(s) = a + 3b s^2 + 5c s^4 = 0), for inputs not too small."""
    disc = np.sqrt(9 * B_ * B_ - 20 * A_ * C_)
    s_max = np.sqrt((-3 * B_ - disc) / (10 * C_))   # local maximum of p
    s_min = np.sqrt((-3 * B_ + disc) / (10 * C_))   # local minimum of p
    hi, lo = float(p_float(s_max)), float(p_float(s_min))
    assert 0.55 < s_max < 0.56 and 1.05 < s_min < 1.06
    # smallest input singular value whose 5-fold image reaches the band (p^5 increasing there)
    lo_s, hi_s = 1e-6, 0.5
    for _ in range(200):
        mid = 0.5 * (lo_s + hi_s)
        lo_s, hi_s = (mid, hi_s) if p_iter(mid, 5) < lo else (lo_s, mid)
    tau = hi_s
    grid = np.linspace(tau, 1.0, 200001)
    img = p_iter(grid, 5)
    assert img.min() >= lo - 1e-12 and img.max() <= hi + 1e-12
    for k, (m, n) in enumerate([(16, 48), (64, 256), (48, 48)]):
        G = _rng(200 + k).standard_normal((m, n))
        O = _ns_normalised(G, 5, eps=0.0)
        s_in = np.linalg.svd(G, compute_uv=False) / np.linalg.norm(G)
        s_out = np.linalg.svd(O, compute_uv=False)
        s_in_sorted = np.sort(s_in)
        mask = s_in_sorted >= tau
        # singular values map monotonically only per value; compare as multisets via p^5
        assert np.allclose(np.sort(s_out), np.sort(p_iter(s_in, 5)), rtol=1e-10, atol=1e-13)
        sel = np.sort(p_iter(s_in_sorted[mask], 5))
        assert sel.min() >= lo - 1e-12 and sel.max() <= hi + 1e-12


def pin_p6_transpose():
    """P6: NS(G^T) = NS(G)^T, and the wide-form route equals the literal route."""
    G = _rng(300).standard_normal((96, 24))
    O_lit = _ns_normalised(G, 5, literal=True)
    O_wide = _ns_normalised(G, 5, literal=False)
    O_t = _ns_normalised(G.T, 5)
    assert _rel(O_wide, O_lit) < 1e-12
    assert _rel(O_t.T, O_lit) < 1e-12


def pin_p7_invariances():
    """P7: scale, sign and orthogonal invariance of the normalised odd iteration."""
    G = _rng(400).standard_normal((12, 20))
    O = _ns_normalised(G, 5)
    assert _rel(_ns_normalised(37.5 * G, 5), O) < 1e-12
    assert _rel(_ns_normalised(-G, 5), -O) < 1e-12
    Q1, _ = np.linalg.qr(_rng(401).standard_normal((12, 12)))
    Q2, _ = np.linalg.qr(_rng(402).standard_normal((20, 20)))
    assert _rel(_ns_normalised(Q1 @ G @ Q2, 5), Q1 @ O @ Q2) < 1e-11


def pin_p8_rank1_and_equal_sigma():
    """P8: rank one -> p^5(1) u v^T; m equal singular values -> p^5(1/sqrt m) G/sigma."""
    r = _rng(500)
    u, v = r.standard_normal(10), r.standard_normal(30)
    G = np.outer(u, v)
    O = _ns_normalised(G, 5, eps=0.0)
    p5_1 = Fraction(1)
    for _ in range(5):
        p5_1 = p_frac(p5_1)
    want = float(p5_1) * np.outer(u / np.linalg.norm(u), v / np.linalg.norm(v))
    assert _rel(O, want) < 1e-12
    for m in (4, 16, 64):
        Q, _ = np.linalg.qr(r.standard_normal((3 * m, m)))
        G = 2.5 * Q.T                         # m x 3m with all singular values 2.5
        O = _ns_normalised(G, 5, eps=0.0)
        assert _rel(O, p_iter(1 / np.sqrt(m), 5) * Q.T) < 1e-11


def pin_p9_momentum_closed_form():
    """P9: M_T = sum_s beta^(T-s) g_s and U_T = g_T + beta M_T (Nesterov), U_T = M_T
    otherwise; with one gradient reused, every O_t is NS5(G/||G||_F) and
    W_3 = W_0 - 3 lr NS5(G/||G||_F)."""
    r = _rng(600)
    beta, lr = 0.95, 0.02
    gs = [r.standard_normal((6, 9)) for _ in range(4)]
    for nesterov in (True, False):
        W = r.standard_normal((6, 9))
        M = np.zeros((6, 9))
        for T in range(1, 5):
            W2, M, O, nu = om.muon_step(W, M, gs[T - 1], lr=lr, beta=beta, nesterov=nesterov)
            M_cf = sum(beta ** (T - s) * gs[s - 1] for s in range(1, T + 1))
            U_cf = gs[T - 1] + beta * M_cf if nesterov else M_cf
            assert np.max(np.abs(M - M_cf)) < 1e-12
            assert abs(nu - np.linalg.norm(U_cf)) < 1e-12 * nu
            assert _rel(O, _ns_normalised(U_cf, 5, eps=om.DEFAULT_EPS)) < 1e-12
            assert np.max(np.abs(W2 - (W - lr * O))) < 1e-15
            W = W2
    # one gradient reused three times (the 64x256 fp32 workload)
    G = r.standard_normal((64, 256))
    W0 = 0.02 * r.standard_normal((64, 256))
    outs = list(om.muon_run(W0, [G, G, G], lr=lr, beta=beta, nesterov=True))
    kappa_m = [1.0, 1.95, 2.8525]
    kappa_u = [1.95, 2.8525, 3.709875]
    M = np.zeros_like(G)
    for t, (W, M, O, nu) in enumerate(outs):
        assert np.max(np.abs(M - kappa_m[t] * G)) < 1e-12
        assert abs(nu - kappa_u[t] * np.linalg.norm(G)) < 1e-9
    O_ref = _ns_normalised(G, 5, eps=0.0)
    assert _rel(outs[-1][0], W0 - 3 * lr * O_ref) < 1e-9


def pin_p10_zero_padding():
    """P10: NS([G 0; 0 0]) = [NS(G) 0; 0 0] (the iteration never mixes in zero rows/cols)."""
    G = _rng(700).standard_normal((7, 11))
    P = np.zeros((16, 24))
    P[:7, :11] = G
    O = om.newton_schulz(G / np.linalg.norm(G), 5)
    OP = om.newton_schulz(P / np.linalg.norm(P), 5)
    assert np.max(np.abs(OP[:7, :11] - O)) < 1e-13
    assert np.max(np.abs(OP[7:, :])) == 0.0 and np.max(np.abs(OP[:, 11:])) == 0.0


def pin_p11_zero_steps():
    """P11: with ns_steps = 0 the update is U / (||U||_F + eps)."""
    r = _rng(800)
    G, W = r.standard_normal((5, 8)), r.standard_normal((5, 8))
    W2, M, O, nu = om.muon_step(W, np.zeros((5, 8)), G, ns_steps=0)
    U = G + 0.95 * G
    assert np.max(np.abs(O - U / (np.linalg.norm(U) + 1e-7))) < 1e-15


def pin_p12_zero_gradient():
    """P12: zero momentum and zero gradient give O = 0 and leave W unchanged; a zero
    gradient on a non-zero buffer decays it by beta."""
    r = _rng(900)
    W = r.standard_normal((4, 6))
    W2, M, O, nu = om.muon_step(W, np.zeros((4, 6)), np.zeros((4, 6)))
    assert nu == 0.0 and np.all(O == 0) and np.all(W2 == W) and np.all(M == 0)
    M0 = r.standard_normal((4, 6))
    _, M1, _, _ = om.muon_step(W, M0, np.zeros((4, 6)))
    assert np.max(np.abs(M1 - 0.95 * M0)) < 1e-15


def pin_p13_brute_force_eig():
    """P13: on <= 8x8 inputs, NS(X) = q(X X^T) X with q(lambda) = p^5(sqrt lambda)/sqrt lambda,
    evaluated through a symmetric eigendecomposition (a route independent of the iteration)."""
    for k, (m, n) in enumerate([(3, 3), (4, 7), (8, 8), (2, 5), (6, 8)]):
        G = _rng(1000 + k).standard_normal((m, n))
        X = G / np.linalg.norm(G)
        lam, V = np.linalg.eigh(X @ X.T)
        s = np.sqrt(np.maximum(lam, 0))
        q = p_iter(s, 5) / s
        want = (V * q) @ V.T @ X
        got = om.newton_schulz(X, 5)
        assert _rel(got, want) < 1e-10, ((m, n), _rel(got, want))


def pin_coefficient_schedule():
    """A per-round (a, b, c) schedule equal to the fixed triple changes nothing, and a
    schedule acts per singular value as the composition of its polynomials."""
    G = _rng(1100).standard_normal((6, 10))
    X = G / np.linalg.norm(G)
    same = om.newton_schulz(X, 3, schedule=[om.DEFAULT_ABC] * 3)
    assert _rel(same, om.newton_schulz(X, 3)) < 1e-15
    sched = [(3.0, -3.2, 1.2), (2.0, -1.5, 0.5), (1.5, -0.5, 0.0)]
    got = om.newton_schulz(X, 3, schedule=sched)
    U, S, Vt = np.linalg.svd(X, full_matrices=False)
    s = S.copy()
    for a, b, c in sched:
        s = a * s + b * s ** 3 + c * s ** 5
    assert _rel(got, (U * s) @ Vt) < 1e-12


ALL_PINS = [
    pin_p1_hand_expansion, pin_p2_diagonal_worked_example, pin_p3_symmetric_2x2,
    pin_p4_svd_identity, pin_p5_band, pin_p6_transpose, pin_p7_invariances,
    pin_p8_rank1_and_equal_sigma, pin_p9_momentum_closed_form, pin_p10_zero_padding,
    pin_p11_zero_steps, pin_p12_zero_gradient, pin_p13_brute_force_eig,
    pin_coefficient_schedule,
]
