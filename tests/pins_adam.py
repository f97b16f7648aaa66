"""Pins: checks of the cautious-Adam oracle against facts that do not come from the oracle.

They use:

* a first step from zero moments worked out by hand: there the bias-corrected moments are
  g and g^2, so with eps = 0 the Adam direction is sign(g) (Kingma and Ba 2015);
* PyTorch's own Adam and AdamW on the CPU in float64, an independent implementation of the
  textbook optimizer, for the moments, the bias correction and the decoupled decay;
* the mask rule of the record analysis at lqnn.cn (section 3.3): decay only where the update
  and the parameter agree in sign; read back from PyTorch's Adam step, not from the oracle;
* symmetries of the step (odd in (p, g, m), invariant to the gradient's scale when eps = 0).

Each pin raises AssertionError when the oracle disagrees. They look up the oracle's
functions through the module at call time, so a test can plant a mistake in the oracle
(monkeypatch) and check that some pin catches it.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle.cautious_adam as oa


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def pin_a1_first_step_by_hand():
    """t = 1 from zero moments, beta1 0.9, beta2 0.999, eps 0, lr 0.1, decay 0.5: u = sign(g).

    element  p      g     u    u*p>0  u + 0.5*mask*p  p - 0.1*(...)
    0        0.5    3     1    yes    1.25            0.375
    1        0.5   -1    -1    no    -1               0.6
    2       -0.25   2     1    no     1              -0.35
    3       -2     -0.5  -1    yes   -2              -1.8
    4        0      1     1    no     1              -0.1
    m = 0.1 g and v = 0.001 g^2.
    """
    p = np.array([0.5, 0.5, -0.25, -2.0, 0.0])
    g = np.array([3.0, -1.0, 2.0, -0.5, 1.0])
    z = np.zeros(5)
    p1, m1, v1, mask = oa.cautious_adam_step(p, g, z, z, 1, 0.1, 0.9, 0.999, 0.0,
                                             weight_decay=0.25, wd_mul=2.0)
    np.testing.assert_allclose(p1, [0.375, 0.6, -0.35, -1.8, -0.1], rtol=0, atol=1e-14)
    np.testing.assert_allclose(m1, 0.1 * g, rtol=1e-14, atol=0)
    np.testing.assert_allclose(v1, 0.001 * g * g, rtol=1e-12, atol=0)
    assert mask.tolist() == [True, False, False, True, False]
    # a zero gradient with eps > 0 gives u = 0: no step and, the comparison being strict,
    # no decay either
    p2, _, _, mask2 = oa.cautious_adam_step(np.array([0.7, -0.3]), np.zeros(2), np.zeros(2),
                                            np.zeros(2), 1, 0.1, 0.9, 0.999, 1e-8,
                                            weight_decay=0.5)
    np.testing.assert_array_equal(p2, [0.7, -0.3])
    assert not mask2.any()


def _torch_step(opt_cls, p, g, m, v, t, lr, b1, b2, eps, wd):
    """One step of a PyTorch optimizer in float64 from the state (p, m, v) after t - 1 steps."""
    P = torch.nn.Parameter(torch.tensor(p, dtype=torch.float64))
    opt = opt_cls([P], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd, foreach=False)
    P.grad = torch.tensor(g, dtype=torch.float64)
    if t > 1:
        opt.state[P] = {"step": torch.tensor(float(t - 1), dtype=torch.float64),
                        "exp_avg": torch.tensor(m, dtype=torch.float64),
                        "exp_avg_sq": torch.tensor(v, dtype=torch.float64)}
    opt.step()
    st = opt.state[P]
    return (P.detach().numpy().copy(), st["exp_avg"].numpy().copy(),
            st["exp_avg_sq"].numpy().copy())


def pin_a2_torch_adam_without_decay():
    """Six steps with decay 0 (and with a multiplier but zero base decay) equal torch Adam."""
    r = _rng(11)
    shape = (7, 13)
    p = r.normal(0, 0.02, shape)
    m = np.zeros(shape)
    v = np.zeros(shape)
    P = torch.nn.Parameter(torch.tensor(p, dtype=torch.float64))
    opt = torch.optim.Adam([P], lr=3e-3, betas=(0.8, 0.95), eps=1e-10, foreach=False)
    for t in range(1, 7):
        g = r.normal(0, 1e-3, shape) * (1 + t)
        p, m, v, _ = oa.cautious_adam_step(p, g, m, v, t, 3e-3, 0.8, 0.95, 1e-10,
                                           weight_decay=0.0, wd_mul=150.0)
        P.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        np.testing.assert_allclose(p, P.detach().numpy(), rtol=1e-12, atol=1e-16)
        np.testing.assert_allclose(m, opt.state[P]["exp_avg"].numpy(), rtol=1e-12, atol=0)
        np.testing.assert_allclose(v, opt.state[P]["exp_avg_sq"].numpy(), rtol=1e-12, atol=0)


def pin_a3_masked_adamw():
    """From states along a trajectory, each element of the oracle's step equals torch AdamW's
    (decay = base * multiplier) where the Adam step and the parameter agree in sign, and torch
    Adam's elsewhere. The mask is read off torch Adam's step direction."""
    r = _rng(12)
    shape = (9, 31)
    lr, b1, b2, eps, wd, mul = 1e-2, 0.9, 0.99, 1e-8, 0.05, 10.0
    p = r.normal(0, 0.5, shape)
    m = np.zeros(shape)
    v = np.zeros(shape)
    both = [0, 0]
    for t in range(1, 5):
        g = r.normal(0, 1.0, shape)
        pa, ma, va = _torch_step(torch.optim.Adam, p, g, m, v, t, lr, b1, b2, eps, 0.0)
        pw, mw, vw = _torch_step(torch.optim.AdamW, p, g, m, v, t, lr, b1, b2, eps, wd * mul)
        direction = (p - pa) / lr                 # torch Adam's bias-corrected direction
        agree = direction * p > 0
        expect = np.where(agree, pw, pa)
        p1, m1, v1, mask = oa.cautious_adam_step(p, g, m, v, t, lr, b1, b2, eps,
                                                 weight_decay=wd, wd_mul=mul)
        np.testing.assert_array_equal(mask, agree)
        np.testing.assert_allclose(p1, expect, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(m1, ma, rtol=1e-12, atol=0)
        np.testing.assert_allclose(v1, va, rtol=1e-12, atol=0)
        np.testing.assert_allclose(mw, ma, rtol=0, atol=0)   # decay never enters the moments
        both[0] += int(agree.sum())
        both[1] += int((~agree).sum())
        p, m, v = p1, m1, v1
    assert min(both) > 100                        # both branches of the mask were exercised


def pin_a4_symmetries():
    """The step is odd in (p, g, m) with v fixed, and with eps = 0 it does not change when
    g, m and v are scaled by (c, c, c^2)."""
    r = _rng(13)
    shape = (5, 40)
    p = r.normal(0, 0.3, shape)
    g = r.normal(0, 1.0, shape)
    m = r.normal(0, 0.3, shape)
    v = r.uniform(0.1, 1.0, shape)
    args = (3, 0.02, 0.9, 0.95, 0.0, 0.4, 1.0)
    p1, m1, v1, mask = oa.cautious_adam_step(p, g, m, v, *args)
    q1, n1, w1, mask_n = oa.cautious_adam_step(-p, -g, -m, v, *args)
    np.testing.assert_allclose(q1, -p1, rtol=1e-13, atol=0)
    np.testing.assert_allclose(n1, -m1, rtol=1e-13, atol=0)
    np.testing.assert_allclose(w1, v1, rtol=1e-13, atol=0)
    np.testing.assert_array_equal(mask_n, mask)
    c = 37.5
    s1, _, _, mask_s = oa.cautious_adam_step(p, c * g, c * m, c * c * v, *args)
    np.testing.assert_allclose(s1, p1, rtol=1e-12, atol=1e-15)
    np.testing.assert_array_equal(mask_s, mask)
    assert mask.any() and not mask.all()


ALL_PINS = [pin_a1_first_step_by_hand, pin_a2_torch_adam_without_decay, pin_a3_masked_adamw,
            pin_a4_symmetries]
