"""The cautious-Adam oracle against its pins, and planted mistakes that the pins must catch
(no GPU). Mistakes are planted on the CPU with monkeypatch; the oracle on disk is untouched."""
import numpy as np
import pytest

import oracle.cautious_adam as oa
import pins_adam


@pytest.mark.parametrize("pin", pins_adam.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def _moments(kind):
    def mom(m, v, g, beta1, beta2):
        if kind == "no_one_minus_beta":
            return beta1 * m + g, beta2 * v + g * g
        if kind == "abs_second_moment":
            return beta1 * m + (1 - beta1) * g, beta2 * v + (1 - beta2) * np.abs(g)
        if kind == "swapped_betas":
            return beta2 * m + (1 - beta2) * g, beta1 * v + (1 - beta1) * (g * g)
        raise ValueError(kind)
    return mom


def _direction(kind):
    def direction(m, v, t, beta1, beta2, eps):
        if kind == "no_bias_correction":
            return m / (np.sqrt(v) + eps)
        if kind == "eps_inside_sqrt":
            return (m / (1 - beta1 ** t)) / np.sqrt(v / (1 - beta2 ** t) + eps)
        if kind == "step_off_by_one":
            return (m / (1 - beta1 ** (t + 1))) / (np.sqrt(v / (1 - beta2 ** (t + 1))) + eps)
        raise ValueError(kind)
    return direction


def _decay(kind):
    def decay(u, p, lam):
        if kind == "mask_reversed":
            mask = (u * p) < 0
        elif kind == "mask_not_strict":
            mask = (u * p) >= 0
        elif kind == "no_mask":
            mask = np.ones(u.shape, dtype=bool)
        elif kind == "minus_decay":
            mask = (u * p) > 0
            return u - lam * np.where(mask, p, 0.0), mask
        else:
            raise ValueError(kind)
        return u + lam * np.where(mask, p, 0.0), mask
    return decay


def _step(kind):
    def step(p, g, m, v, t, lr, beta1, beta2, eps, weight_decay=0.0, wd_mul=1.0):
        p, g, m, v = (np.array(x, dtype=np.float64) for x in (p, g, m, v))
        lam = weight_decay * wd_mul
        if kind == "coupled_decay":                 # L2 penalty folded into the gradient
            mask = (p * g) > 0
            g = g + lam * np.where(mask, p, 0.0)
            lam = 0.0
        m, v = oa.adam_moments(m, v, g, beta1, beta2)
        u = oa.adam_direction(m, v, t, beta1, beta2, eps)
        if kind == "mask_on_gradient":
            mask = (g * p) > 0
            u = u + lam * np.where(mask, p, 0.0)
        elif kind == "decay_not_scaled_by_lr":
            u0 = u
            u, mask = oa.cautious_decay(u, p, lam)
            return p - lr * u0 - (u - u0), m, v, mask
        elif kind == "base_decay_only":
            u, mask = oa.cautious_decay(u, p, weight_decay)
        else:
            u, mask = oa.cautious_decay(u, p, lam)
        return p - lr * u, m, v, mask
    return step


MUTANTS = {
    "moments_no_one_minus_beta": ("adam_moments", _moments("no_one_minus_beta")),
    "moments_abs_second": ("adam_moments", _moments("abs_second_moment")),
    "moments_swapped_betas": ("adam_moments", _moments("swapped_betas")),
    "direction_no_bias_correction": ("adam_direction", _direction("no_bias_correction")),
    "direction_eps_inside_sqrt": ("adam_direction", _direction("eps_inside_sqrt")),
    "direction_step_off_by_one": ("adam_direction", _direction("step_off_by_one")),
    "decay_mask_reversed": ("cautious_decay", _decay("mask_reversed")),
    "decay_mask_not_strict": ("cautious_decay", _decay("mask_not_strict")),
    "decay_no_mask": ("cautious_decay", _decay("no_mask")),
    "decay_minus": ("cautious_decay", _decay("minus_decay")),
    "step_coupled_decay": ("cautious_adam_step", _step("coupled_decay")),
    "step_mask_on_gradient": ("cautious_adam_step", _step("mask_on_gradient")),
    "step_decay_not_scaled_by_lr": ("cautious_adam_step", _step("decay_not_scaled_by_lr")),
    "step_base_decay_only": ("cautious_adam_step", _step("base_decay_only")),
}


def _failing_pins():
    failed = []
    for pin in pins_adam.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    return failed


def test_unmutated_oracle_passes_all_pins():
    assert _failing_pins() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(monkeypatch, name):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oa, attr, fn)
    with np.errstate(all="ignore"):
        failed = _failing_pins()
    assert failed, f"no pin catches the planted mistake {name}"


def test_adam_sets_seeded():
    import seeded_inputs as si
    s = si.ADAM_SETS["gpt2_124m_embed"]
    assert s.elements() == 4 * 50257 * 768 + 64
    assert [t[2] for t in s.tensors] == [150.0, 1.0, 1.0, 1.0, 0.0]
    r = si.ADAM_SETS["ragged_small"]
    a, b = si.adam_grad(r, 7, 2), si.adam_grad(r, 7, 2)
    assert bool((a == b).all()) and not bool((a == si.adam_grad(r, 7, 3)).all())
    assert abs(float(si.adam_param(r, 7).std()) - 0.5) < 0.01
