"""The library's per-launch timing (muon_plan_set_profiling / muon_plan_read_profile) on the
GPU: it does not change results, counts every kernel of a step, and its durations (taken
from the kernel dispatches themselves) fit inside the wall time of the steps they cover."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from orthogonalized_momentum_optimizer_amd import MuonPlan, make_config

pytestmark = pytest.mark.gpu

SHAPES = [(768, 768)] * 6 + [(768, 3072), (3072, 768)] * 3   # two shape groups, 3 launch sets


def _run(profile, steps=3):
    dev = torch.device("cuda", 0)
    wl = si.custom(SHAPES, dtype="bf16", steps=steps, cfg_id=120)
    W = [si.weight(wl, i).to(dev) for i in range(wl.n)]
    M = [torch.zeros(s, dtype=torch.float32, device=dev) for s in wl.shapes]
    O = [torch.empty(s, dtype=torch.float32, device=dev) for s in wl.shapes]
    G = [[si.grad(wl, i, t).to(dev) for i in range(wl.n)] for t in range(steps)]
    plan = MuonPlan(wl.shapes, [w.dtype for w in W], [w.dtype for w in W], "bf16", dev)
    cfg = make_config()
    plan.set_profiling(profile)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(steps):
        plan.step(W, G[t], M, cfg, outs=O)
    e1.record()
    torch.cuda.synchronize()
    wall_ms = e0.elapsed_time(e1)
    prof = plan.read_profile()
    plan.set_profiling(False)
    after = plan.read_profile()
    plan.step(W, G[0], M, cfg, outs=O)      # untimed: the totals stay cleared
    torch.cuda.synchronize()
    after2 = plan.read_profile()
    plan.close()
    res = [[x.double().cpu().numpy() for x in (W[i], M[i], O[i])] for i in range(wl.n)]
    return res, prof, wall_ms, after, after2


def test_profiling_counts_and_timing():
    print("[gpu] per-launch timing", flush=True)
    steps = 3
    base, _, _, _, _ = _run(False, steps)
    res, prof, wall_ms, after, after2 = _run(True, steps)
    # timing changes nothing in the results
    for a, b in zip(base, res):
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
    # every kind of the step ran and was timed
    for kind in ("momentum", "norm", "gram", "poly", "apply", "update"):
        ms, n = prof[kind]
        assert n > 0 and ms > 0.0, (kind, prof[kind])
    assert prof["roweq"] == (0.0, 0)
    # one Gram, polynomial and apply launch per round and launch of the products
    ng, npoly, na = prof["gram"][1], prof["poly"][1], prof["apply"][1]
    assert ng == npoly == na and ng % (5 * steps) == 0
    # the elementwise phases: at least one launch per launch set and step
    assert prof["momentum"][1] >= steps and prof["update"][1] >= steps
    # dispatch-timed kernel durations fit in the wall time of the timed steps
    total = sum(ms for ms, _ in prof.values())
    assert total <= wall_ms * 1.02, (total, wall_ms)
    # disabling clears the totals, and untimed steps add nothing
    assert all(v == (0.0, 0) for v in after.values())
    assert all(v == (0.0, 0) for v in after2.values())
