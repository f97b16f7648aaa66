"""Float64 reference of the Muon step, written step by step from the pages.

TEST INFRASTRUCTURE ONLY (see the package docstring). Pure numpy; every input is upcast
exactly to float64 and every operation runs in float64 with numpy's matmul.

The step, per matrix (W: weights, M: momentum buffer, G: gradient):

1. Momentum [P3 "核心算法": "standard SGD momentum" with defaults momentum=0.95,
   nesterov=True]:  M <- beta*M + G;  U = G + beta*M (Nesterov) or U = M.
2. Frobenius pre-normalisation [P4 §3.2 names it; P3's printed iteration omits it]:
   nu = ||U||_F;  X = U / (nu + eps).
3. Wide form: if rows > cols, X <- X^T (the iteration of step 4 commutes with
   transposition, so this changes nothing in exact arithmetic).
4. Quintic Newton-Schulz [P3 "Newton-Schulz正交化"], ns_steps rounds with
   (a, b, c) = (3.4445, -4.7750, 2.0315). A round is the odd quintic p(s) = a s + b s^3 +
   c s^5 applied to every singular value of X: X <- a X + b (X X^T) X + c (X X^T)^2 X,
   evaluated here as q(X X^T) X with q(t) = a + t (b + c t) (Horner's rule).
5. Back to the original orientation: O = X (or X^T if step 3 transposed).
6. Parameter update [P3 "核心算法", third phase of ``step``]:  W <- W - lr * O.

Readings of what the pages leave open (each is a plain choice, recorded here):

* R1 normalisation in front of the iteration, by the Frobenius norm, eps = 1e-7.
* R3 momentum form without dampening (M <- beta M + G) and Nesterov U = G + beta M.
* R6 the update is lr * O with no shape factor and no weight decay.
* The oracle does not round to bf16: the pages' bf16 cast is the precision the GPU
  path is measured in, not part of what the method computes.
"""
from __future__ import annotations

from typing import Iterable, Sequence, Tuple

import numpy as np

# [P3 "Newton-Schulz正交化"]: the three coefficients of the quintic iteration.
DEFAULT_ABC = (3.4445, -4.7750, 2.0315)
DEFAULT_EPS = 1e-7


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):                      # a torch tensor (bf16 has no numpy dtype)
        x = x.detach().cpu().double().numpy()
    return np.array(x, dtype=np.float64, copy=True)


def momentum_update(M: np.ndarray, G: np.ndarray, beta: float, nesterov: bool
                    ) -> Tuple[np.ndarray, np.ndarray]:
    """[P3 "核心算法"] SGD momentum: returns (new M, the vector U that is orthogonalised)."""
    M_new = beta * M + G
    U = G + beta * M_new if nesterov else M_new.copy()
    return M_new, U


def frobenius_normalize(U: np.ndarray, eps: float = DEFAULT_EPS) -> Tuple[np.ndarray, float]:
    """[P4 §3.2, reading R1] X = U / (||U||_F + eps); also returns nu = ||U||_F.

    The norm is the square root of the sum of squares (numpy's pairwise summation)."""
    nu = float(np.sqrt(np.sum(U * U)))
    return U / (nu + eps), nu


def newton_schulz(X: np.ndarray, steps: int, abc: Sequence[float] = DEFAULT_ABC,
                  schedule: Sequence[Sequence[float]] | None = None) -> np.ndarray:
    """[P3 "Newton-Schulz正交化"] ``steps`` rounds of the quintic map on X.

    One round maps X = U S V^T to U p(S) V^T with p(s) = a s + b s^3 + c s^5, the odd
    quintic whose coefficients the page prints. Because X X^T = U S^2 U^T, that is
    p(X) = q(X X^T) X with q(t) = a + b t + c t^2, and q of the m x m Gram matrix is
    formed by Horner's rule, q(G) = a I + G (b I + c G), then applied to X.

    ``X`` is used as given (no transposition, no normalisation). ``schedule``, if given,
    holds one (a, b, c) triple per round in place of the fixed ``abc``."""
    X = np.array(X, dtype=np.float64, copy=True)
    eye = np.eye(X.shape[0])
    for k in range(steps):
        a, b, c = schedule[k] if schedule is not None else abc
        gram = X @ X.T                                  # X X^T, the Gram matrix
        q_of_gram = a * eye + gram @ (b * eye + c * gram)   # q(X X^T), Horner's rule
        X = q_of_gram @ X
    return X


def orthogonalize(U: np.ndarray, steps: int, abc: Sequence[float] = DEFAULT_ABC,
                  eps: float = DEFAULT_EPS, literal: bool = False,
                  schedule: Sequence[Sequence[float]] | None = None) -> Tuple[np.ndarray, float]:
    """Steps 2-5 of the module docstring: O = NS(U / (||U||_F + eps)), returned in U's
    orientation, plus nu. ``literal=True`` skips the wide-form transposition."""
    X, nu = frobenius_normalize(np.asarray(U, dtype=np.float64), eps)
    tall = (X.shape[0] > X.shape[1]) and not literal
    if tall:
        X = X.T
    X = newton_schulz(X, steps, abc, schedule)
    return (X.T if tall else X), nu


def muon_step(W, M, G, lr: float = 0.02, beta: float = 0.95, nesterov: bool = True,
              ns_steps: int = 5, abc: Sequence[float] = DEFAULT_ABC, eps: float = DEFAULT_EPS,
              literal: bool = False, schedule=None):
    """One Muon step on one matrix. Returns (W_new, M_new, O, nu), all float64."""
    W, M, G = _f64(W), _f64(M), _f64(G)
    M_new, U = momentum_update(M, G, beta, nesterov)
    O, nu = orthogonalize(U, ns_steps, abc, eps, literal, schedule)
    W_new = W - lr * O
    return W_new, M_new, O, nu


def muon_run(W0, grads: Iterable, **kw):
    """Several Muon steps on one matrix from zero momentum; yields (W, M, O, nu) per step."""
    W = _f64(W0)
    M = np.zeros_like(W)
    for G in grads:
        W, M, O, nu = muon_step(W, M, G, **kw)
        yield W, M, O, nu
