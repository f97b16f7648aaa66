"""Plant plausible mistakes in the CPU oracle and check that some pin catches each one.

The mistakes are planted on the CPU, in the oracle module, with monkeypatch; the oracle on
disk is untouched. A mistake that no pin catches would mean the pins leave that part of
the oracle unchecked.
"""
import numpy as np
import pytest

import oracle.muon as om
import pins


def _ns_factory(kind):
    """The oracle's round X <- q(X X^T) X, q(t) = a + t (b + c t), with one mistake."""
    def ns(X, steps, abc=om.DEFAULT_ABC, schedule=None):
        X = np.array(X, dtype=np.float64, copy=True)
        eye = np.eye(X.shape[0])
        n_rounds = steps + 1 if kind == "extra_round" else steps
        for k in range(n_rounds):
            a, b, c = schedule[k] if schedule is not None and k < len(schedule) else abc
            if kind == "swap_bc":
                b, c = c, b
            if kind == "sign_b":
                b = -b
            gram = X.T @ X if kind == "gram_transposed" else X @ X.T
            if gram.shape[0] != X.shape[0]:       # X^T X only composes for square X
                gram = X @ X.T + 1e-3
            if kind == "linear_c":                # c t in place of c t^2
                q = a * eye + gram * (b + c)
            else:
                q = a * eye + gram @ (b * eye + c * gram)
            if kind == "drop_aX":
                q = q - a * eye
            X = q @ X
        return X
    return ns


def _momentum_factory(kind):
    def mom(M, G, beta, nesterov):
        if kind == "ema":
            M_new = beta * M + (1 - beta) * G
        else:
            M_new = beta * M + G
        if kind == "ignore_nesterov":
            U = M_new.copy()
        elif kind == "old_buffer":
            U = G + beta * M if nesterov else M_new.copy()
        else:
            U = G + beta * M_new if nesterov else M_new.copy()
        return M_new, U
    return mom


def _norm_factory(kind):
    def norm(U, eps=om.DEFAULT_EPS):
        if kind == "spectral":
            nu = float(np.linalg.norm(U, 2)) if U.size else 0.0
        elif kind == "max_abs":
            nu = float(np.abs(U).max()) if U.size else 0.0
        elif kind == "squared":
            nu = float(np.sum(U * U))
        else:
            nu = float(np.sqrt(np.sum(U * U)))
        return U / (nu + eps), nu
    return norm


def _orth_no_back_transpose(U, steps, abc=om.DEFAULT_ABC, eps=om.DEFAULT_EPS, literal=False,
                            schedule=None):
    X, nu = om.frobenius_normalize(np.asarray(U, dtype=np.float64), eps)
    tall = X.shape[0] > X.shape[1] and not literal
    if tall:
        X = X.T
    X = om.newton_schulz(X, steps, abc, schedule)
    if tall:                                   # forgets to transpose back: flips and reshapes
        X = X.T[::-1].copy()
    return X, nu


def _step_factory(kind):
    orig = om.muon_step

    def step(W, M, G, lr=0.02, beta=0.95, nesterov=True, ns_steps=5, abc=om.DEFAULT_ABC,
             eps=om.DEFAULT_EPS, literal=False, schedule=None):
        W2, M2, O, nu = orig(W, M, G, lr, beta, nesterov, ns_steps, abc, eps, literal, schedule)
        W = om._f64(W)
        if kind == "plus_sign":
            W2 = W + lr * O
        elif kind == "no_lr":
            W2 = W - O
        return W2, M2, O, nu
    return step


MUTANTS = {
    "ns_swap_bc": ("newton_schulz", _ns_factory("swap_bc")),
    "ns_sign_b": ("newton_schulz", _ns_factory("sign_b")),
    "ns_gram_transposed": ("newton_schulz", _ns_factory("gram_transposed")),
    "ns_linear_c": ("newton_schulz", _ns_factory("linear_c")),
    "ns_drop_aX": ("newton_schulz", _ns_factory("drop_aX")),
    "ns_extra_round": ("newton_schulz", _ns_factory("extra_round")),
    "mom_ema": ("momentum_update", _momentum_factory("ema")),
    "mom_ignore_nesterov": ("momentum_update", _momentum_factory("ignore_nesterov")),
    "mom_old_buffer": ("momentum_update", _momentum_factory("old_buffer")),
    "norm_spectral": ("frobenius_normalize", _norm_factory("spectral")),
    "norm_max_abs": ("frobenius_normalize", _norm_factory("max_abs")),
    "norm_squared": ("frobenius_normalize", _norm_factory("squared")),
    "orth_no_back_transpose": ("orthogonalize", _orth_no_back_transpose),
    "step_plus_sign": ("muon_step", _step_factory("plus_sign")),
    "step_no_lr": ("muon_step", _step_factory("no_lr")),
}


def _failing_pins():
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError, np.linalg.LinAlgError):
            failed.append(pin.__name__)
    return failed


def test_unmutated_oracle_passes_all_pins():
    assert _failing_pins() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(monkeypatch, name):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(om, attr, fn)
    with np.errstate(all="ignore"):
        failed = _failing_pins()
    assert failed, f"no pin catches the planted mistake {name}"
