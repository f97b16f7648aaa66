"""The row-equaliser oracle against its pins, and planted mistakes that the pins must catch
(no GPU). Mistakes are planted on the CPU with monkeypatch; the oracle on disk is untouched."""
import numpy as np
import pytest

import oracle.muon as om
import oracle.row_equalizer as oe
import pins_roweq


@pytest.mark.parametrize("pin", pins_roweq.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def _moment(kind):
    def mom(O, v, beta2):
        if kind == "columns":
            ms = np.mean(O * O, axis=0)
            ms = np.resize(ms, v.shape)
        elif kind == "rms_not_squared":
            ms = np.sqrt(np.mean(O * O, axis=1))
        else:
            ms = np.mean(O * O, axis=1)
        if kind == "swapped_beta":
            return (1.0 - beta2) * v + beta2 * ms
        if kind == "no_state":
            return ms
        return beta2 * v + (1.0 - beta2) * ms
    return mom


def _equalize(kind):
    def eq(O, v, beta2=oe.DEFAULT_ROW_BETA, eps=oe.DEFAULT_ROW_EPS):
        O = np.asarray(O, dtype=np.float64)
        v_new = oe.row_second_moment(O, np.asarray(v, dtype=np.float64), beta2)
        if kind == "no_sqrt":
            D = O / (v_new[:, None] + eps)
        elif kind == "eps_inside_sqrt":
            D = O / np.sqrt(v_new[:, None] + eps)
        elif kind == "old_state":
            D = O / (np.sqrt(np.asarray(v, dtype=np.float64))[:, None] + eps + 1e-300)
        else:
            D = O / (np.sqrt(v_new)[:, None] + eps)
        if kind == "no_rescale":
            return D, v_new
        if kind == "rescale_to_rows":
            return D * np.sqrt(O.shape[0]) / np.linalg.norm(D), v_new
        e_o, e_d = np.linalg.norm(O), np.linalg.norm(D)
        return (D * (e_o / e_d) if e_d > 0 else np.zeros_like(O)), v_new
    return eq


MUTANTS = {
    "moment_columns": ("row_second_moment", _moment("columns")),
    "moment_rms_not_squared": ("row_second_moment", _moment("rms_not_squared")),
    "moment_swapped_beta": ("row_second_moment", _moment("swapped_beta")),
    "moment_no_state": ("row_second_moment", _moment("no_state")),
    "equalize_no_sqrt": ("row_equalize", _equalize("no_sqrt")),
    "equalize_eps_inside_sqrt": ("row_equalize", _equalize("eps_inside_sqrt")),
    "equalize_old_state": ("row_equalize", _equalize("old_state")),
    "equalize_no_rescale": ("row_equalize", _equalize("no_rescale")),
    "equalize_rescale_to_rows": ("row_equalize", _equalize("rescale_to_rows")),
}


def _failing_pins():
    failed = []
    for pin in pins_roweq.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError, ZeroDivisionError):
            failed.append(pin.__name__)
    return failed


def test_unmutated_oracle_passes_all_pins():
    assert _failing_pins() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(monkeypatch, name):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oe, attr, fn)
    with np.errstate(all="ignore"):
        failed = _failing_pins()
    assert failed, f"no pin catches the planted mistake {name}"


def test_equalized_step_composes_the_muon_step():
    """The equalised step is the Muon step with O replaced by its equalised form: same
    momentum, same orthogonalisation (checked against oracle.muon_step), W - lr O'."""
    r = np.random.Generator(np.random.PCG64(24))
    W, G = r.normal(0, 0.02, (20, 9)), r.normal(0, 1e-3, (20, 9))
    M, V = r.normal(0, 1e-3, (20, 9)), r.uniform(0, 1e-3, 20)
    W1, M1, O, nu = om.muon_step(W, M, G)
    W2, M2, V2, O2, nu2 = oe.muon_step_equalized(W, M, V, G)
    O_ref, V_ref = oe.row_equalize(O, V)
    np.testing.assert_array_equal(M2, M1)
    assert nu2 == nu
    np.testing.assert_allclose(O2, O_ref, rtol=1e-15)
    np.testing.assert_allclose(V2, V_ref, rtol=1e-15)
    np.testing.assert_allclose(W2, W - 0.02 * O_ref, rtol=1e-15)
    # zero gradient and momentum: W unchanged, the state decays
    W3, _, V3, O3, _ = oe.muon_step_equalized(W, np.zeros_like(W), V, np.zeros_like(W))
    np.testing.assert_array_equal(W3, W)
    np.testing.assert_allclose(V3, 0.95 * V, rtol=1e-15)
