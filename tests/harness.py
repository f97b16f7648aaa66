"""Shared helpers of the GPU parity tests: run seeded workloads through the library and
through the CPU oracle, and compare them."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import seeded_inputs as si
from orthogonalized_momentum_optimizer_amd import MuonPlan, make_config

TOL = {"bf16": 3e-2, "f32": 1e-4}        # relative Frobenius error of O and W
# A weight stored in bf16 carries a relative rounding of up to 2^-9 per element after
# every update, whatever the precision of the Newton-Schulz rounds; such weights are
# compared at the bf16 tolerance, weights stored in fp32 at the tolerance of the rounds.
M_TOL = 1e-6                             # momentum: max |dM| / max |M| (fp32 buffer)

_TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def rel(x: np.ndarray, y: np.ndarray) -> float:
    d = np.linalg.norm(y)
    return float(np.linalg.norm(x - y) / d) if d > 0 else float(np.linalg.norm(x))


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().double().cpu().numpy()


def gpu_fill_grad(wl, i, t, dev):
    """Seeded gradient drawn on the GPU (for matrices whose values the test never compares)."""
    g = torch.Generator(device=dev)
    g.manual_seed(1_000_003 * wl.cfg_id + 7919 * i + t + 17)
    r, c = wl.shapes[i]
    return (wl.grad_std * torch.randn(r, c, generator=g, device=dev)).to(_TORCH_DT[wl.dtype])


def run_gpu(wl, steps, precision="bf16", watch=None, cfg=None, gpu_fill_others=False,
            grads=None, dev=None, W0=None):
    """Runs ``steps`` Muon steps of workload ``wl`` on the GPU. Returns, for every matrix in
    ``watch`` (default: all), per-step float64 copies of (W, M, O)."""
    dev = dev or torch.device("cuda", 0)
    n = wl.n
    watch = list(range(n)) if watch is None else list(watch)
    cfg = cfg or make_config()
    def w_init(i):
        if W0 is not None:
            return W0[i].to(dev)
        if gpu_fill_others and i not in watch:
            return (0.02 / wl.grad_std) * gpu_fill_grad(wl, i, 10_000, dev).float()
        return si.weight(wl, i).to(dev)

    W = [w_init(i) for i in range(n)]
    W = [w.to(_TORCH_DT[wl.dtype]) for w in W]
    M = [torch.zeros(s, dtype=torch.float32, device=dev) for s in wl.shapes]
    O = [torch.empty(s, dtype=torch.float32, device=dev) if i in watch else None
         for i, s in enumerate(wl.shapes)]
    plan = MuonPlan(wl.shapes, [w.dtype for w in W], [w.dtype for w in W], precision, dev)
    out = {i: [] for i in watch}
    for t in range(steps):
        if grads is not None:
            G = [grads[i][t].to(dev) for i in range(n)]
        else:
            G = [(si.grad(wl, i, t).to(dev) if (i in watch or not gpu_fill_others)
                  else gpu_fill_grad(wl, i, t, dev)) for i in range(n)]
        plan.step(W, G, M, cfg, outs=O)
        torch.cuda.synchronize()
        for i in watch:
            out[i].append((f64(W[i]), f64(M[i]), f64(O[i])))
    plan.close()
    return out


def run_oracle(wl, i, steps, grads=None, **kw):
    gs = [grads[i][t] if grads is not None else si.grad(wl, i, t) for t in range(steps)]
    return [(W, M, O) for W, M, O, _ in oracle.muon_run(si.weight(wl, i), gs, **kw)]


def compare(wl, gpu, steps, precision, grads=None, report=None, oracle_kw=None):
    """Element-by-element comparison of every watched matrix and step with the oracle.
    Returns the worst (O error, W error, M error)."""
    tol = TOL[precision]
    w_tol = max(tol, TOL["bf16"]) if wl.dtype == "bf16" else tol
    worst = [0.0, 0.0, 0.0]
    for i, traj in gpu.items():
        ref = run_oracle(wl, i, steps, grads=grads, **(oracle_kw or {}))
        for t, ((Wg, Mg, Og), (Wr, Mr, Or)) in enumerate(zip(traj, ref)):
            eo, ew = rel(Og, Or), rel(Wg, Wr)
            mmax = np.max(np.abs(Mr))
            em = float(np.max(np.abs(Mg - Mr)) / mmax) if mmax > 0 else float(np.max(np.abs(Mg)))
            worst = [max(worst[0], eo), max(worst[1], ew), max(worst[2], em)]
            if report is not None:
                report.append((i, t, eo, ew, em))
            assert eo <= tol, f"matrix {i} {wl.shapes[i]} step {t}: O rel err {eo:.3e} > {tol}"
            assert ew <= w_tol, f"matrix {i} step {t}: W rel err {ew:.3e} > {w_tol}"
            assert em <= M_TOL, f"matrix {i} step {t}: M rel err {em:.3e} > {M_TOL}"
    print(f"{wl.name} [{precision}] worst O {worst[0]:.3e}  W {worst[1]:.3e}  M {worst[2]:.3e}",
          flush=True)
    return worst
