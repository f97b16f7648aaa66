"""Float64 reference of the per-row energy equaliser applied to the orthogonalised update.

TEST INFRASTRUCTURE ONLY (see the package docstring). Pure numpy in float64.

Source: the RecursiveFromBest record analysis (lqnn.cn/news/184262), section 3.2 "NorMuon
中的退火行 RMS 缩放 Langevin/SGLD 探索噪声": the NorMuon-family optimizer of that record
follows the orthogonalisation with a per-lane energy equaliser taken from NorMuon, built on a
low-rank, Adafactor-style estimate of the update's variance. The page prints no formula;
the readings below are the plainest ones its description supports:

* N1 a lane is a row of the matrix in its own orientation (one output unit of the weight),
  whatever orientation the iteration ran in;
* N2 the variance estimate is a rank-1 (per-row) exponential moving average of the mean
  square of the orthogonalised update O: v_i <- beta2 v_i + (1 - beta2) mean_j O_ij^2,
  kept in an fp32 state buffer of one value per row (zero before the first step);
* N3 each row is divided by its estimated RMS: D_ij = O_ij / (sqrt(v_i) + eps); with
  eps = 0 a row whose state is 0 (its O row, a mean of squares, is then all zero) stays 0;
* N4 an energy equaliser moves energy between lanes without changing the total: the result
  is D rescaled to O's Frobenius norm, O'_ij = D_ij ||O||_F / ||D||_F (0 when O is 0);
  a uniform factor on v (such as a bias correction) therefore cancels, up to eps;
* N5 the parameter update uses O' in place of O: W <- W - lr O'.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from . import muon as om

DEFAULT_ROW_BETA = 0.95
DEFAULT_ROW_EPS = 1e-8


def row_second_moment(O: np.ndarray, v: np.ndarray, beta2: float) -> np.ndarray:
    """[N1, N2] The per-row EMA of the mean square of O."""
    return beta2 * v + (1.0 - beta2) * np.mean(O * O, axis=1)


def row_equalize(O, v, beta2: float = DEFAULT_ROW_BETA, eps: float = DEFAULT_ROW_EPS
                 ) -> Tuple[np.ndarray, np.ndarray]:
    """[N2-N4] Returns (O', v') for an update O (rows x cols) and the row state v (rows)."""
    O = np.asarray(O, dtype=np.float64)
    v_new = row_second_moment(O, np.asarray(v, dtype=np.float64), beta2)
    den = np.sqrt(v_new)[:, None] + eps
    # [N3] a row whose denominator is 0 has v' = 0, so the row of O is zero and stays zero
    D = np.divide(O, den, out=np.zeros_like(O), where=den > 0)
    e_o = float(np.sqrt(np.sum(O * O)))
    e_d = float(np.sqrt(np.sum(D * D)))
    return (D * (e_o / e_d) if e_d > 0 else np.zeros_like(O)), v_new


def muon_step_equalized(W, M, V, G, lr: float = 0.02, beta: float = 0.95,
                        nesterov: bool = True, ns_steps: int = 5, abc=om.DEFAULT_ABC,
                        eps: float = om.DEFAULT_EPS, row_beta: float = DEFAULT_ROW_BETA,
                        row_eps: float = DEFAULT_ROW_EPS, schedule=None):
    """One Muon step with the row equaliser between the orthogonalisation and the update
    [N5]. Returns (W_new, M_new, V_new, O', nu), all float64."""
    W, M, G = om._f64(W), om._f64(M), om._f64(G)
    M_new, U = om.momentum_update(M, G, beta, nesterov)
    O, nu = om.orthogonalize(U, ns_steps, abc, eps, schedule=schedule)
    O_eq, V_new = row_equalize(O, V, row_beta, row_eps)
    return W - lr * O_eq, M_new, V_new, O_eq, nu


def muon_run_equalized(W0, grads, **kw):
    """Several equalised Muon steps from zero momentum and zero row state; yields
    (W, M, V, O', nu) per step."""
    W = om._f64(W0)
    M = np.zeros_like(W)
    V = np.zeros(W.shape[0])
    for G in grads:
        W, M, V, O, nu = muon_step_equalized(W, M, V, G, **kw)
        yield W, M, V, O, nu
