"""muon_step_noalloc, the entry point whose kernels use the library's static device scratch
instead of a caller's workspace, against muon_step on the same inputs, through the C ABI.

Two calls in a row on the static scratch, the second with a smaller input: the 8-GPU share of
the GPT-2-124M set (61.2 MiB of scratch, near its 64 MiB limit), then a small ragged set (a few
hundred KiB, so most of the scratch still holds the first call's values). Both entry points
run the same kernels on the same inputs, so W, M and O must agree bitwise; one matrix of each
call is also compared with the float64 oracle at the bf16 tolerances. A third call runs the
row equaliser through the static scratch.
"""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from harness import compare
from orthogonalized_momentum_optimizer_amd import MuonPlan, make_config

pytestmark = pytest.mark.gpu


def _run(wl, steps, noalloc, cfg=None, row_eq=False):
    dev = torch.device("cuda", 0)
    W = [si.weight(wl, i).to(dev) for i in range(wl.n)]
    M = [torch.zeros(s, dtype=torch.float32, device=dev) for s in wl.shapes]
    O = [torch.empty(s, dtype=torch.float32, device=dev) for s in wl.shapes]
    V = [torch.zeros(s[0], dtype=torch.float32, device=dev) for s in wl.shapes] if row_eq else None
    plan = MuonPlan(wl.shapes, [w.dtype for w in W], [w.dtype for w in W], "bf16", dev,
                    workspace=not noalloc)
    cfg = cfg or make_config()
    out = {i: [] for i in range(wl.n)}
    for t in range(steps):
        G = [si.grad(wl, i, t).to(dev) for i in range(wl.n)]
        if noalloc:
            plan.step_noalloc(W, G, M, cfg, outs=O, row_vars=V)
        else:
            plan.step(W, G, M, cfg, outs=O, row_vars=V)
        torch.cuda.synchronize()
        for i in range(wl.n):
            out[i].append(tuple(x.double().cpu().numpy() for x in (W[i], M[i], O[i])))
    plan.close()
    return out


def _same(a, b, label):
    for i in a:
        for t, (x, y) in enumerate(zip(a[i], b[i])):
            for k in range(3):
                assert np.array_equal(x[k], y[k]), f"{label}: matrix {i} step {t} field {k}"


def test_noalloc_matches_step_on_two_calls_in_a_row():
    share = si.WORKLOADS["gpt2_124m_share8"]
    small = si.custom([(200, 328), (328, 200), (96, 160)], dtype="bf16", steps=2, cfg_id=150)
    print("[gpu] noalloc: reference runs with a workspace", flush=True)
    ref_big = _run(share, 2, noalloc=False)
    ref_small = _run(small, 2, noalloc=False)
    print("[gpu] noalloc: share8 then the small set on the static scratch", flush=True)
    got_big = _run(share, 2, noalloc=True)
    got_small = _run(small, 2, noalloc=True)
    _same(ref_big, got_big, "gpt2_124m_share8")
    _same(ref_small, got_small, "small set")
    compare(share, {0: got_big[0], 6: got_big[6]}, 2, "bf16")
    compare(small, {1: got_small[1]}, 2, "bf16")


def test_noalloc_row_equalizer_matches_step():
    wl = si.custom([(384, 256), (256, 640)], dtype="bf16", steps=2, cfg_id=151)
    cfg = make_config(row_equalize=True)
    print("[gpu] noalloc: row equaliser", flush=True)
    _same(_run(wl, 2, False, cfg, row_eq=True), _run(wl, 2, True, cfg, row_eq=True), "roweq")


def test_noalloc_single_launch_rounds_match_step():
    """A set that takes the single-launch rounds (three 256-aligned groups of 8 matrices, 20.5
    MiB of scratch): its queues and completion counters then live in the static scratch and
    are cleared by the launch's own clearing kernel on every call."""
    wl = si.custom([(256, 256)] * 8 + [(512, 256)] * 8 + [(256, 1024)] * 8, dtype="bf16",
                   steps=2, cfg_id=152)
    print("[gpu] noalloc: single-launch rounds", flush=True)
    _same(_run(wl, 2, False), _run(wl, 2, True), "single-launch rounds")
