"""The parity harness itself, on the CPU: its bf16 storage model, the W gate derived from it,
and the choice of watched matrices. A simulated GPU trajectory (the oracle's O with fp32-
sized noise, the update in fp32 arithmetic stored in bf16 by torch) must pass every gate,
and planted storage mistakes must fail the bf16-storage W gate although they pass the 3e-2
gate against the exact trajectory."""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from harness import StepChecker, bf16_round


def test_bf16_round_matches_torch_on_float32_values():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-30, 30, 200_000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(bf16_round(x.astype(np.float64)), ref)


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 (bf16 spacing 2^-7 on [1, 2)): even is 1;
    # 1 + 3 * 2^-8 lies between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 0.0, 2.0 ** -100])
    assert list(bf16_round(x)) == [1.0, 1 + 2.0 ** -6, -1.0, 0.0, 2.0 ** -100]
    ref = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(bf16_round(x), ref)


def _simulated_gpu(wl, i, steps, rounding="nearest", lr_gpu=0.02, noise=2e-6, seed=0):
    """The oracle's O plus relative noise of size ``noise`` (what fp32 rounds leave), the
    momentum in fp32, and the update computed in fp32 and stored in bf16."""
    rng = np.random.default_rng(seed)
    W = si.weight(wl, i).float()
    M = np.zeros(wl.shapes[i])
    out = []
    for t in range(steps):
        G = si.grad(wl, i, t)
        _, M, O, _ = oracle.muon_step(W, M, G)
        Og = O + noise * np.linalg.norm(O) / np.sqrt(O.size) * rng.standard_normal(O.shape)
        y = W - lr_gpu * torch.from_numpy(Og).float()
        if rounding == "nearest":
            W = y.to(torch.bfloat16).float()
        else:  # truncation toward zero: the low 16 bits of the fp32 value dropped
            W = (y.view(torch.int32) & ~0xFFFF).view(torch.float32)
        out.append((G, W.double().numpy(), np.float32(M).astype(np.float64),
                    np.float32(Og).astype(np.float64)))
    return out


WL = si.custom([(96, 160)], dtype="bf16", steps=10, cfg_id=130)


def _run_checker(traj):
    chk = StepChecker("sim", si.weight(WL, 0), "bf16", "f32", 0.02)
    worst = 0.0
    for G, Wg, Mg, Og in traj:
        eo, ew, em, es = chk.check(G, Wg, Mg, Og)
        worst = max(worst, es)
    return worst, ew


def test_storage_gate_accepts_a_faithful_trajectory():
    worst, _ = _run_checker(_simulated_gpu(WL, 0, 10))
    assert worst < 1e-3


@pytest.mark.parametrize("mistake", ["truncating store", "lr 1% off"])
def test_storage_gate_rejects_storage_mistakes(mistake):
    kw = {"truncating store": dict(rounding="truncate"), "lr 1% off": dict(lr_gpu=0.0202)}
    traj = _simulated_gpu(WL, 0, 10, **kw[mistake])
    with pytest.raises(AssertionError, match="W~"):
        _run_checker(traj)
    # the exact-trajectory gate of the bf16 tolerance alone would have let it through
    chk = StepChecker("sim", si.weight(WL, 0), "bf16", "bf16", 0.02)
    for G, Wg, Mg, Og in traj:
        chk.check(G, Wg, Mg, Og)


def test_row_outliers_are_row_dominated():
    """The tall-stress trajectory test watches the tall and the wide matrix whose step-0
    gradient has the largest share of its energy in one row; their rows do dominate."""
    from test_gpu_trajectories import _row_outliers
    wl = si.WORKLOADS["tall_stress"]
    idx = _row_outliers(wl)
    assert len(idx) == 2 and wl.shapes[idx[0]] != wl.shapes[idx[1]]
    for i in idx:
        g = si.grad(wl, i, 0).double().numpy()
        rows = (g * g).sum(axis=1)
        assert rows.max() / rows.sum() > 0.2
