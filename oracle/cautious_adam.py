"""Float64 reference of one cautious-Adam step over a tensor of any shape.

TEST INFRASTRUCTURE ONLY (see the package docstring). Pure numpy in float64.

Source: the RecursiveFromBest record analysis (lqnn.cn/news/184262), section 3.3 "bigram 与
value-embedding 银行上的 C-Optim / 谨慎 Adam". The record moves the embedding-like parameters
(bigram table, value-embedding banks, embed / lm_head) to an Adam whose weight decay is
"cautious": decay is applied to an element only where the Adam update and the parameter have
the same sign, which the page states as a mask (update * p > 0) and a masked addition of
p times an effective decay to the update. The same section's parameter table gives each
tensor a decay multiplier (150 for embed and lm_head, 0 for scalars).

The step, per element (p parameter, g gradient, m and v the two moment buffers, t >= 1 the
index of this step):

1. Moments (textbook Adam, Kingma and Ba 2015, the optimizer the page names):
   m <- beta1 m + (1 - beta1) g;   v <- beta2 v + (1 - beta2) g^2.
2. Direction with bias correction: u = (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps).
3. Cautious decay [section 3.3]: mask = (u * p > 0);  u <- u + lam * mask * p, with
   lam = weight_decay * wd_mul.
4. Update: p <- p - lr * u.

Readings of what the page leaves open (each a plain choice, recorded here):

* A1 the moments and the bias correction are textbook Adam; the page prints neither.
* A2 the effective decay is the base decay times the tensor's multiplier; the page names an
  effective decay without its formula.
* A3 the decay is decoupled (it never enters m or v) and is scaled by lr together with the
  Adam direction, so with every mask element set the step is AdamW's and with none set it
  is Adam's; the mask compares the direction u with the parameter before the step.
* A4 the comparison is strict: an element with u = 0 or p = 0 is not decayed.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):                      # a torch tensor (bf16 has no numpy dtype)
        x = x.detach().cpu().double().numpy()
    return np.array(x, dtype=np.float64, copy=True)


def adam_moments(m: np.ndarray, v: np.ndarray, g: np.ndarray, beta1: float, beta2: float
                 ) -> Tuple[np.ndarray, np.ndarray]:
    """[A1] The two exponential moving averages of Adam: of g and of g squared."""
    return beta1 * m + (1.0 - beta1) * g, beta2 * v + (1.0 - beta2) * (g * g)


def adam_direction(m: np.ndarray, v: np.ndarray, t: int, beta1: float, beta2: float,
                   eps: float) -> np.ndarray:
    """[A1] Bias-corrected Adam direction of step t (t counts from 1)."""
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    return m_hat / (np.sqrt(v_hat) + eps)


def cautious_decay(u: np.ndarray, p: np.ndarray, lam: float) -> Tuple[np.ndarray, np.ndarray]:
    """[section 3.3, A3, A4] Adds lam * p to the direction where u and p agree in sign.
    Returns (new direction, mask)."""
    mask = (u * p) > 0
    return u + lam * np.where(mask, p, 0.0), mask


def cautious_adam_step(p, g, m, v, t: int, lr: float, beta1: float, beta2: float, eps: float,
                       weight_decay: float = 0.0, wd_mul: float = 1.0):
    """One step on one tensor. Returns (p', m', v', mask) as float64 arrays of p's shape."""
    if t < 1:
        raise ValueError("t counts from 1")
    p, g, m, v = _f64(p), _f64(g), _f64(m), _f64(v)
    m, v = adam_moments(m, v, g, beta1, beta2)
    u = adam_direction(m, v, t, beta1, beta2, eps)
    u, mask = cautious_decay(u, p, weight_decay * wd_mul)
    return p - lr * u, m, v, mask


def cautious_adam_run(p0, grads, lr: float, beta1: float, beta2: float, eps: float,
                      weight_decay: float = 0.0, wd_mul: float = 1.0, t0: int = 1):
    """Steps t0, t0+1, ... with the given gradients from zero moments; returns the list of
    per-step (p, m, v, mask)."""
    p = _f64(p0)
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    out = []
    for k, g in enumerate(grads):
        p, m, v, mask = cautious_adam_step(p, g, m, v, t0 + k, lr, beta1, beta2, eps,
                                           weight_decay, wd_mul)
        out.append((p.copy(), m.copy(), v.copy(), mask.copy()))
    return out
