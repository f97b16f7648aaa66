"""The CPU oracle against its pins (no GPU)."""
import numpy as np
import pytest

import pins
import seeded_inputs as si


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_seeded_inputs_deterministic():
    wl = si.WORKLOADS["gpt2_tiny_fp32"]
    a, b = si.grad(wl, 0, 0), si.grad(wl, 0, 2)
    assert a.dtype == b.dtype and bool((a == b).all())          # reused gradient
    w1, w2 = si.weight(wl, 0), si.weight(wl, 0)
    assert bool((w1 == w2).all())
    wl2 = si.WORKLOADS["attn_768"]
    g0, g1 = si.grad(wl2, 0, 0), si.grad(wl2, 0, 1)
    assert not bool((g0 == g1).all())
    assert abs(float(g0.float().std()) - 1e-3) < 2e-5
    assert abs(float(si.weight(wl2, 0).float().std()) - 0.02) < 2e-4


def test_workload_inventory():
    w = si.WORKLOADS
    assert w["gpt2_124m"].n == 72 and w["gpt2_124m"].elements() == 84_934_656
    assert w["tall_stress"].elements() == 226_492_416
    assert w["gpt2_1p5b"].n == 288 and w["gpt2_1p5b"].elements() == 1_474_560_000
    # nominal Newton-Schulz flops of one step (4 m^2 n + 2 m^3 per round, m <= n)
    assert abs(w["gpt2_124m"].ns_flops_per_step() / 1e9 - 1630.7) < 0.1
    assert abs(w["attn_768"].ns_flops_per_step() / 1e9 - 13.59) < 0.01


def test_heavy_tailed_rows():
    wl = si.custom([(512, 64)], heavy_tailed_rows=True, cfg_id=3)
    g = si.grad(wl, 0, 0).float().numpy()
    rms = np.sqrt((g ** 2).mean(axis=1))
    assert rms.max() / np.median(rms) > 5       # Student-t(3) row scales are heavy tailed


def test_iid_student_t_entries():
    wl = si.custom([(512, 64)], iid_t3_entries=True, cfg_id=4)
    g = si.grad(wl, 0, 0).float().numpy()
    a = np.abs(g).ravel()
    # Student-t(3) entries: far heavier tails than a Gaussian of the same median size
    assert a.max() / np.median(a) > 15
    # but no row scaling: the row energies stay within a modest range of each other
    rms = np.sqrt((g ** 2).mean(axis=1))
    assert np.median(rms) > 0 and rms.min() / np.median(rms) > 0.3
