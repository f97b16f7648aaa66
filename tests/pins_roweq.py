"""Pins: checks of the row-equaliser oracle against facts that do not come from the oracle.

They use hand-worked 2x2 cases (first step from a zero state; a later step from a given
state, with and without eps), the closed form of the first step (every row of the result
carries the same energy, ||O||_F^2 / rows, along the caller's rows), a matrix whose rows
already have equal energy (unchanged), equivariance under row permutations and a positive
scale, and the zero update. The equaliser is the per-lane energy equaliser named in the
record analysis at lqnn.cn (section 3.2); the readings are listed in the oracle's header.

Each pin raises AssertionError when the oracle disagrees; the oracle's functions are looked
up through the module at call time so that tests can plant mistakes in it.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import oracle.row_equalizer as oe


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def pin_e1_first_step_by_hand():
    """O = [[3, 4], [0, 1]], zero state, beta2 0.95, eps 0: the rows (norms 5 and 1) are
    scaled to equal energy 13 each (||O||^2 = 26): [[0.6, 0.8], [0, 1]] * sqrt(13); the state
    becomes 0.05 * (12.5, 0.5)."""
    O2, v = oe.row_equalize(np.array([[3.0, 4.0], [0.0, 1.0]]), np.zeros(2), 0.95, 0.0)
    r13 = np.sqrt(13.0)
    np.testing.assert_allclose(O2, [[0.6 * r13, 0.8 * r13], [0.0, r13]], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(v, [0.625, 0.025], rtol=1e-14)


def pin_e2_later_step_by_hand():
    """beta2 0.75, state (7/24, 7/6), O = [[0.3, 0.4], [0.6, 0.8]] (row mean squares 1/8 and
    1/2): v' = 0.75 v + 0.25 ms = (1/4, 1). With eps 0 the rows divide by (1/2, 1), giving
    [[0.6, 0.8], [0.6, 0.8]] (energy 2), rescaled to ||O||^2 = 5/4: factor sqrt(5/8). With
    eps = 1/2 they divide by (1, 3/2): [[0.3, 0.4], [0.4, 8/15]] (energy 25/36), factor
    sqrt((5/4) / (25/36)) = sqrt(9/5)."""
    v0 = np.array([float(Fraction(7, 24)), float(Fraction(7, 6))])
    O = np.array([[0.3, 0.4], [0.6, 0.8]])
    O2, v = oe.row_equalize(O, v0, 0.75, 0.0)
    np.testing.assert_allclose(v, [0.25, 1.0], rtol=1e-14)
    np.testing.assert_allclose(O2, np.array([[0.6, 0.8], [0.6, 0.8]]) * np.sqrt(5 / 8),
                               rtol=1e-13)
    O3, _ = oe.row_equalize(O, v0, 0.75, 0.5)
    np.testing.assert_allclose(O3, np.array([[0.3, 0.4], [0.4, 8 / 15]]) * np.sqrt(9 / 5),
                               rtol=1e-13)


def pin_e3_first_step_equal_row_energy():
    """From a zero state with eps 0 every row of the result has energy ||O||_F^2 / rows, the
    rows being the caller's rows (tall and wide shapes), and the total energy is kept."""
    r = _rng(21)
    for shape in ((40, 7), (7, 40), (33, 33)):
        O = r.normal(0, 1, shape) * r.uniform(0.1, 3.0, (shape[0], 1))
        O2, _ = oe.row_equalize(O, np.zeros(shape[0]), 0.9, 0.0)
        e = np.sum(O * O)
        np.testing.assert_allclose(np.sum(O2 * O2, axis=1), e / shape[0], rtol=1e-12)
        # directions within a row are kept
        np.testing.assert_allclose(O2 / np.linalg.norm(O2, axis=1, keepdims=True),
                                   O / np.linalg.norm(O, axis=1, keepdims=True), rtol=1e-12)


def pin_e4_equal_rows_unchanged_and_energy_kept():
    """An orthogonal matrix (rows of equal energy) is unchanged at the first step; from any
    state the Frobenius norm is kept."""
    r = _rng(22)
    Q, _ = np.linalg.qr(r.normal(0, 1, (24, 24)))
    O2, _ = oe.row_equalize(Q, np.zeros(24), 0.95, 0.0)
    np.testing.assert_allclose(O2, Q, rtol=1e-12, atol=1e-14)
    O = r.normal(0, 1, (16, 50))
    v = r.uniform(0.0, 2.0, 16)
    O3, _ = oe.row_equalize(O, v, 0.8, 1e-3)
    np.testing.assert_allclose(np.linalg.norm(O3), np.linalg.norm(O), rtol=1e-13)


def pin_e5_equivariance():
    """Permuting rows (with the state) permutes the result; scaling O by c > 0 and the state
    by c^2 scales the result by c (eps 0)."""
    r = _rng(23)
    O = r.normal(0, 1, (12, 30))
    v = r.uniform(0.1, 1.0, 12)
    base, vb = oe.row_equalize(O, v, 0.9, 0.0)
    perm = r.permutation(12)
    Op, vp = oe.row_equalize(O[perm], v[perm], 0.9, 0.0)
    np.testing.assert_allclose(Op, base[perm], rtol=1e-13)
    np.testing.assert_allclose(vp, vb[perm], rtol=1e-14)
    c = 7.25
    Oc, vc = oe.row_equalize(c * O, c * c * v, 0.9, 0.0)
    np.testing.assert_allclose(Oc, c * base, rtol=1e-12)
    np.testing.assert_allclose(vc, c * c * vb, rtol=1e-13)


def pin_e6_zero_update():
    """A zero update stays zero and the state decays by beta2; with eps 0, a zero row with a
    zero state stays zero while the other rows keep all the energy: [[3, 4], [0, 0]] is
    unchanged."""
    O2, v = oe.row_equalize(np.zeros((3, 5)), np.array([1.0, 2.0, 0.0]), 0.9, 1e-8)
    assert not O2.any()
    np.testing.assert_allclose(v, [0.9, 1.8, 0.0], rtol=1e-15)
    O3, v3 = oe.row_equalize(np.array([[3.0, 4.0], [0.0, 0.0]]), np.zeros(2), 0.95, 0.0)
    np.testing.assert_allclose(O3, [[3.0, 4.0], [0.0, 0.0]], rtol=1e-14, atol=0)
    np.testing.assert_allclose(v3, [0.625, 0.0], rtol=1e-14)


ALL_PINS = [pin_e1_first_step_by_hand, pin_e2_later_step_by_hand,
            pin_e3_first_step_equal_row_energy, pin_e4_equal_rows_unchanged_and_energy_kept,
            pin_e5_equivariance, pin_e6_zero_update]
