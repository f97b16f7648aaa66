"""All Newton-Schulz rounds as one persistent launch (muon_plan_set_fused, on by default).
It computes the per-product kernels' products in their order with their instructions, so a
step with it must give bitwise the W, momentum and O of the same step with one launch per
product; parity with the oracle over whole trajectories is in test_gpu_trajectories.py (the
GPT-2-124M set takes this launch by default). Round counts 1 and 2 check the
ping-pong of X (the result lands in either buffer), 16 the largest the launch takes; a
per-round coefficient table checks that each round reads its own (a, b, c)."""
import pytest
import torch

import seeded_inputs as si
from orthogonalized_momentum_optimizer_amd import MuonPlan, make_config

pytestmark = pytest.mark.gpu


def dev():
    return torch.device("cuda", 0)


# three shape groups of 8 matrices, 256-aligned: 256x256, 512x256 (tall, runs as 256x512) and
# 256x1024; with 8 matrices per group every XCD holds one matrix of each
SMALL = [(256, 256)] * 8 + [(512, 256)] * 8 + [(256, 1024)] * 8
# two groups of 768-row matrices (the GPT-2-124M widths at a sixth of its count): 768x768 and
# 1536x768 (tall, runs as 768x1536)
MID = [(768, 768)] * 8 + [(1536, 768)] * 8
# four groups, the most the launch takes: 256x256, 256x768, 512x512 and 1024x512 (tall, runs as
# 512x1024), with 8, 9, 16 and 11 matrices (a group whose count is not a multiple of 8 leaves
# some XCDs one matrix fewer), interleaved in the list
FOUR = ([(256, 256), (256, 768), (512, 512), (1024, 512)] * 8 + [(256, 768), (512, 512)]
        + [(512, 512)] * 7 + [(1024, 512)] * 3)


def _error_flag(plan, wl):
    """The single launch's error flag (set when a wait for a matrix's inputs gave up): the
    workspace ends with its queues (8 x 16 words), the flag, 15 spare words and the completion
    counters (3 x 16 rounds words per matrix), 256-byte aligned."""
    words = 8 * 16 + 16 + 3 * 16 * wl.n
    off = plan.ws_bytes - (4 * words + 255) // 256 * 256
    return int(plan.workspace[off + 512:off + 516].cpu().view(torch.int32)[0])


def _steps(wl, fused, cfg, steps, dtype=torch.bfloat16, scale=1.0, single=None):
    """W, M and O after `steps` steps; W and G in `dtype` (the rounds are bf16 either way),
    the seeded gradients multiplied by `scale`. The library's launch counts confirm which path
    ran (`single`, by default `fused`): the single launch once per step, or no single launch
    and one launch per product."""
    single = fused if single is None else single
    plan = MuonPlan(wl.shapes, [dtype] * wl.n, [dtype] * wl.n, "bf16", dev(), fused=fused)
    plan.set_profiling(True)
    W = [si.weight(wl, i).to(dev(), dtype) for i in range(wl.n)]
    M = [torch.zeros(s, dtype=torch.float32, device=dev()) for s in wl.shapes]
    O = [torch.empty(s, dtype=torch.float32, device=dev()) for s in wl.shapes]
    for t in range(steps):
        G = [(si.grad(wl, i, t).float() * scale).to(dev(), dtype) for i in range(wl.n)]
        plan.step(W, G, M, cfg, outs=O)
        torch.cuda.synchronize()
        if single:
            assert _error_flag(plan, wl) == 0, f"step {t}: a wait of the single launch gave up"
    prof = plan.read_profile()
    if single:
        assert prof["rounds"][1] == steps and prof["apply"][1] == 0, prof
    else:
        assert prof["rounds"][1] == 0 and prof["apply"][1] > 0, prof
    out = [x.clone() for x in W + M + O]
    plan.close()
    return out


def _assert_bitwise(a, b, what):
    bad = [i for i, (x, y) in enumerate(zip(a, b)) if not torch.equal(x, y)]
    assert not bad, f"{what}: buffers {bad[:10]} differ between the single launch and per-product launches"


@pytest.mark.parametrize("ns_steps", [1, 2, 5, 16])
def test_single_launch_rounds_equal_per_product_launches(ns_steps):
    print(f"[fused] small set, ns_steps={ns_steps}", flush=True)
    wl = si.custom(SMALL, steps=2, cfg_id=150 + ns_steps)
    cfg = make_config(ns_steps=ns_steps)
    _assert_bitwise(_steps(wl, True, cfg, 2), _steps(wl, False, cfg, 2), f"ns_steps {ns_steps}")


@pytest.mark.parametrize("ns_steps", [1, 3, 5])
def test_single_launch_768_rows_equal_per_product_launches(ns_steps):
    print(f"[fused] 768-row set, ns_steps={ns_steps}", flush=True)
    wl = si.custom(MID, steps=3, cfg_id=160 + ns_steps)
    cfg = make_config(ns_steps=ns_steps)
    _assert_bitwise(_steps(wl, True, cfg, 3), _steps(wl, False, cfg, 3), f"ns_steps {ns_steps}")


@pytest.mark.parametrize("ns_steps", [2, 5])
def test_single_launch_four_groups_equal_per_product_launches(ns_steps):
    print(f"[fused] four groups, ns_steps={ns_steps}", flush=True)
    wl = si.custom(FOUR, steps=2, cfg_id=180 + ns_steps)
    cfg = make_config(ns_steps=ns_steps)
    _assert_bitwise(_steps(wl, True, cfg, 2), _steps(wl, False, cfg, 2), f"ns_steps {ns_steps}")


@pytest.mark.parametrize("scale,eps", [(1e-22, 0.0), (1e-22, 1e-7), (1e22, 1e-7)])
def test_single_launch_extreme_gradient_scales(scale, eps):
    """Gradient entries near 1e-25 and 1e19: the norm kernel rescales X_0 by a power of two
    before the rounds (its fp32 Gram accumulation would underflow or overflow otherwise), and
    the single launch then runs on the rescaled X_0 with the adjusted s1. Bitwise the per-
    product launches' result, and O finite (with eps = 1e-7 the small gradients' O is the
    rounds applied to U / eps, small but not zero)."""
    print(f"[fused] small set, gradient scale {scale:g}, eps {eps:g}", flush=True)
    wl = si.custom(SMALL, steps=2, cfg_id=190)
    cfg = make_config(eps=eps)
    fused = _steps(wl, True, cfg, 2, scale=scale)
    _assert_bitwise(fused, _steps(wl, False, cfg, 2, scale=scale), f"scale {scale:g}")
    O = fused[2 * wl.n:]
    assert all(bool(torch.isfinite(o).all()) and bool(o.abs().max() > 0) for o in O)


def test_more_rounds_than_the_single_launch_takes():
    """17 rounds, one more than the launch's round table holds: a plan with the single launch
    enabled runs one launch per product instead, with the same results."""
    print("[fused] small set, ns_steps=17: one launch per product", flush=True)
    wl = si.custom(SMALL, steps=1, cfg_id=195)
    cfg = make_config(ns_steps=17)
    _assert_bitwise(_steps(wl, True, cfg, 1, single=False), _steps(wl, False, cfg, 1),
                    "ns_steps 17")


def test_single_launch_fp32_parameters_and_gradients():
    print("[fused] small set, fp32 W and G", flush=True)
    wl = si.custom(SMALL, steps=2, cfg_id=158)
    cfg = make_config()
    _assert_bitwise(_steps(wl, True, cfg, 2, torch.float32),
                    _steps(wl, False, cfg, 2, torch.float32), "fp32 W and G")


def test_single_launch_rounds_with_a_coefficient_table():
    print("[fused] small set, per-round coefficients", flush=True)
    wl = si.custom(SMALL, steps=2, cfg_id=170)
    g = torch.Generator().manual_seed(170)
    u = (torch.rand(5, 3, generator=g) * 2 - 1).tolist()
    # a different (a, b, c) every round, of the size of the fixed map's
    table = [(3.0 + 0.5 * a, -4.5 + 0.5 * b, 2.0 + 0.25 * c) for a, b, c in u]
    cfg = make_config(schedule=table)
    _assert_bitwise(_steps(wl, True, cfg, 2), _steps(wl, False, cfg, 2), "schedule")


def test_single_launch_rounds_gpt2_124m_bitwise():
    print("[fused] gpt2_124m, 2 steps", flush=True)
    wl = si.WORKLOADS["gpt2_124m"]
    cfg = make_config()
    _assert_bitwise(_steps(wl, True, cfg, 2), _steps(wl, False, cfg, 2), "gpt2_124m")


def test_single_launch_newton_schulz_entry():
    """muon_newton_schulz (rounds only, no momentum or update) on a set that takes the single
    launch: bitwise the per-product launches' output, and within the bf16 tolerance of the
    oracle's orthogonalisation on one matrix of each group."""
    import numpy as np
    import oracle
    print("[fused] newton_schulz entry, small set", flush=True)
    wl = si.custom(SMALL, cfg_id=175)
    X = [si.grad(wl, i, 0).to(dev()) for i in range(wl.n)]
    outs = []
    for fused in (True, False):
        Y = [torch.empty(s, dtype=torch.float32, device=dev()) for s in wl.shapes]
        plan = MuonPlan(wl.shapes, [torch.float32] * wl.n, [x.dtype for x in X], "bf16", dev(),
                        fused=fused)
        plan.newton_schulz(X, Y, make_config(ns_steps=5))
        torch.cuda.synchronize()
        plan.close()
        outs.append(Y)
    _assert_bitwise(outs[0], outs[1], "newton_schulz")
    for i in (0, 8, 16):
        ref, _ = oracle.orthogonalize(X[i].double().cpu().numpy(), 5)
        got = outs[0][i].double().cpu().numpy()
        err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert err <= 3e-2, (i, err)


def test_single_launch_failure_makes_the_step_nan(monkeypatch):
    """The failure path, forced from the host: with MUON_FUSED_MAX_POLLS=0 (read when a plan is
    made) every wait of the single launch gives up at once, as a stalled device would make it
    do after its poll limit. The launch still ends (its items compute from whatever their
    inputs hold, all in bounds), sets its error flag, and the step's update writes NaN to
    every W and O instead of leaving silently wrong parameters. A plan made afterwards, without
    the variable, steps normally."""
    print("[fused] forced failure of the single launch", flush=True)
    wl = si.custom(SMALL, steps=1, cfg_id=176)
    cfg = make_config()
    monkeypatch.setenv("MUON_FUSED_MAX_POLLS", "0")
    plan = MuonPlan(wl.shapes, [torch.bfloat16] * wl.n, [torch.bfloat16] * wl.n, "bf16", dev())
    monkeypatch.delenv("MUON_FUSED_MAX_POLLS")
    W = [si.weight(wl, i).to(dev()) for i in range(wl.n)]
    M = [torch.zeros(s, dtype=torch.float32, device=dev()) for s in wl.shapes]
    O = [torch.empty(s, dtype=torch.float32, device=dev()) for s in wl.shapes]
    G = [si.grad(wl, i, 0).to(dev()) for i in range(wl.n)]
    plan.step(W, G, M, cfg, outs=O)
    torch.cuda.synchronize()
    assert _error_flag(plan, wl) != 0
    assert all(bool(torch.isnan(w).all()) for w in W)
    assert all(bool(torch.isnan(o).all()) for o in O)
    plan.close()
    # the next plan steps normally
    out = _steps(wl, True, cfg, 1)
    assert all(bool(torch.isfinite(x).all()) for x in out)


def test_single_launch_long_run_bitwise():
    """Many steps in a row (the GPT-2-124M set, 60 steps): two plans that take the single
    launch and one with per-product launches step the same inputs; W, M and O agree bitwise
    after every step. The single launch's items run in an order that changes from run to run,
    so this checks that no ordering of its producers and consumers changes a result."""
    print("[fused] gpt2_124m, 60 steps, two single-launch plans against per-product", flush=True)
    wl = si.WORKLOADS["gpt2_124m"]
    cfg = make_config()
    G = [[si.grad(wl, i, t).to(dev()) for i in range(wl.n)] for t in range(2)]
    runs = []
    for fused in (True, True, False):
        plan = MuonPlan(wl.shapes, [torch.bfloat16] * wl.n, [torch.bfloat16] * wl.n, "bf16",
                        dev(), fused=fused)
        W = [si.weight(wl, i).to(dev()) for i in range(wl.n)]
        M = [torch.zeros(s, dtype=torch.float32, device=dev()) for s in wl.shapes]
        O = [torch.empty(s, dtype=torch.float32, device=dev()) for s in wl.shapes]
        runs.append((plan, W, M, O))
    for t in range(60):
        for plan, W, M, O in runs:
            plan.step(W, G[t % 2], M, cfg, outs=O)
        torch.cuda.synchronize()
        ref = runs[2][1] + runs[2][2] + runs[2][3]
        for k in (0, 1):
            got = runs[k][1] + runs[k][2] + runs[k][3]
            _assert_bitwise(got, ref, f"step {t}, single-launch plan {k}")
    for k in (0, 1):
        assert _error_flag(runs[k][0], wl) == 0
    for plan, *_ in runs:
        plan.close()
