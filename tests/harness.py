"""Shared helpers of the GPU parity tests: run seeded workloads through the library and
through the CPU oracle, and compare them.

Tolerances (relative Frobenius error per matrix and step, against the float64 oracle):

* O (the orthogonalised update, read back through ``update_out``): 3e-2 when the
  Newton-Schulz rounds run in bf16, 1e-4 when they run in fp32 (the fp32 debug precision).
* M (fp32 momentum buffer): max |dM| / max |M| <= 1e-6.
* W stored in fp32: the tolerance of the rounds (3e-2 or 1e-4).
* W stored in bf16: 3e-2 against the oracle's exact trajectory in both precisions (each
  update is rounded to a bf16 grid whose spacing is 2^-8 to 2^-7 of the value). In the fp32
  rounds it is also checked against the oracle's trajectory as bf16 storage leaves it,
  W~_t = bf16(W~_(t-1) - lr O_t), at a bound derived from that storage (``w_storage_bound``).
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import seeded_inputs as si
from orthogonalized_momentum_optimizer_amd import MuonPlan, make_config

TOL = {"bf16": 3e-2, "f32": 1e-4}        # relative Frobenius error of O and W
M_TOL = 1e-6                             # momentum: max |dM| / max |M| (fp32 buffer)
STORAGE_MARGIN = 3.0                     # w_storage_bound: margin over the expected size

_TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def rel(x: np.ndarray, y: np.ndarray) -> float:
    d = np.linalg.norm(y)
    return float(np.linalg.norm(x - y) / d) if d > 0 else float(np.linalg.norm(x))


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().double().cpu().numpy()


def bf16_round(x) -> np.ndarray:
    """float64 values rounded to the nearest bfloat16 value (8 significant bits, ties to
    even), computed exactly in float64: x = m 2^e with 1/2 <= |m| < 1, and m 2^8 rounded to
    an integer by np.rint (half to even). Meant for values in bf16's normal range."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def w_storage_bound(terms: float) -> float:
    """Bound on ||W_gpu - W~||_F after the steps whose terms add up to ``terms``.

    Per element, both sides round to the same bf16 grid: the GPU rounds y = W - lr O_gpu
    (fp32 arithmetic), the storage model rounds y~ = W~ - lr O_ref (exact). Where their
    stored values agree, the two roundings differ only if a rounding boundary lies between
    y and y~, which for a value placed uniformly in its cell happens with probability
    |y - y~| / ulp and then costs one ulp. With |y - y~| <= lr |dO| + (fp32 rounding of the
    update, two roundings of 2^-24) and ulp(x) <= 2^-7 |x| (8 significant bits), the
    expected square of the difference after the steps is at most

        sum_s  (lr ||dO_s|| + 2^-23 ||W~_s||) * 2^-7 ||W~_s||      (Cauchy-Schwarz)

    with ||dO_s|| <= 1e-4 ||O_s|| (the fp32 gate on O). The difference is a count of
    one-ulp flips, so it is compared at STORAGE_MARGIN times the square root of that sum
    (a margin of 9 on the expected count)."""
    return STORAGE_MARGIN * math.sqrt(max(terms, 0.0))


class StepChecker:
    """The oracle's trajectory of one matrix, advanced one step at a time from W0 and zero
    momentum, and the checks of one GPU step against it."""

    def __init__(self, label, W0, w_dtype: str, precision: str, lr: float, oracle_kw=None):
        self.label = label
        self.W = f64(W0)
        self.M = np.zeros_like(self.W)
        self.Wst = self.W.copy()          # the oracle's trajectory stored in bf16
        self.w_dtype, self.precision, self.lr = w_dtype, precision, lr
        self.kw = dict(oracle_kw or {})
        self.kw.setdefault("lr", lr)
        self.terms = 0.0
        self.t = 0
        self.storage_check = w_dtype == "bf16" and precision == "f32"

    def check(self, G, Wg, Mg, Og):
        """G: this step's gradient (stored dtype); Wg, Mg, Og: the GPU's W, M, O after it.
        Returns (O error, W error, M error, W error against the bf16-stored trajectory or
        None) and asserts every gate."""
        self.W, self.M, Or, _ = oracle.muon_step(self.W, self.M, G, **self.kw)
        tol = TOL[self.precision]
        w_tol = TOL["bf16"] if self.w_dtype == "bf16" else tol
        eo, ew = rel(Og, Or), rel(Wg, self.W)
        mmax = np.max(np.abs(self.M))
        em = float(np.max(np.abs(Mg - self.M)) / mmax) if mmax > 0 else float(np.max(np.abs(Mg)))
        where = f"{self.label} step {self.t}"
        assert eo <= tol, f"{where}: O rel err {eo:.3e} > {tol}"
        assert ew <= w_tol, f"{where}: W rel err {ew:.3e} > {w_tol}"
        assert em <= M_TOL, f"{where}: M rel err {em:.3e} > {M_TOL}"
        es = None
        if self.storage_check:
            lr = self.kw["lr"]
            nW = float(np.linalg.norm(self.Wst))
            self.terms += (lr * TOL["f32"] * float(np.linalg.norm(Or)) + 2.0 ** -23 * nW) \
                * 2.0 ** -7 * nW
            self.Wst = bf16_round(self.Wst - lr * Or)
            d = float(np.linalg.norm(Wg - self.Wst))
            bound = w_storage_bound(self.terms)
            es = d / float(np.linalg.norm(self.Wst))
            assert d <= bound, (f"{where}: ||W - W~|| = {d:.3e} > {bound:.3e} "
                                f"(relative {es:.3e} > {bound / np.linalg.norm(self.Wst):.3e})")
        self.t += 1
        return eo, ew, em, es


def gpu_fill_grad(wl, i, t, dev):
    """Seeded gradient drawn on the GPU (for matrices whose values the test never compares)."""
    g = torch.Generator(device=dev)
    g.manual_seed(1_000_003 * wl.cfg_id + 7919 * i + t + 17)
    r, c = wl.shapes[i]
    return (wl.grad_std * torch.randn(r, c, generator=g, device=dev)).to(_TORCH_DT[wl.dtype])


def _init_buffers(wl, watch, dev, gpu_fill_others, W0):
    def w_init(i):
        if W0 is not None:
            return W0[i].to(dev)
        if gpu_fill_others and i not in watch:
            return (0.02 / wl.grad_std) * gpu_fill_grad(wl, i, 10_000, dev).float()
        return si.weight(wl, i).to(dev)

    W = [w_init(i).to(_TORCH_DT[wl.dtype]) for i in range(wl.n)]
    M = [torch.zeros(s, dtype=torch.float32, device=dev) for s in wl.shapes]
    O = [torch.empty(s, dtype=torch.float32, device=dev) if i in watch else None
         for i, s in enumerate(wl.shapes)]
    return W, M, O


def run_gpu(wl, steps, precision="bf16", watch=None, cfg=None, gpu_fill_others=False,
            grads=None, dev=None, W0=None):
    """Runs ``steps`` Muon steps of workload ``wl`` on the GPU. Returns, for every matrix in
    ``watch`` (default: all), per-step float64 copies of (W, M, O)."""
    dev = dev or torch.device("cuda", 0)
    n = wl.n
    watch = list(range(n)) if watch is None else list(watch)
    cfg = cfg or make_config()
    W, M, O = _init_buffers(wl, watch, dev, gpu_fill_others, W0)
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


def _summary(name, precision, worst):
    s = (f"{name} [{precision}] worst O {worst[0]:.3e}  W {worst[1]:.3e}  M {worst[2]:.3e}")
    if worst[3] is not None:
        s += f"  W vs bf16-stored trajectory {worst[3]:.3e}"
    print(s, flush=True)


def _merge(worst, errs):
    eo, ew, em, es = errs
    w = [max(worst[0], eo), max(worst[1], ew), max(worst[2], em), worst[3]]
    if es is not None:
        w[3] = es if w[3] is None else max(w[3], es)
    return w


def compare(wl, gpu, steps, precision, grads=None, report=None, oracle_kw=None):
    """Element-by-element comparison of every watched matrix and step with the oracle.
    Returns the worst (O error, W error, M error, W error against the bf16-stored
    trajectory or None)."""
    kw = dict(oracle_kw or {})
    lr = kw.pop("lr", 0.02)
    worst = [0.0, 0.0, 0.0, None]
    for i, traj in gpu.items():
        chk = StepChecker(f"matrix {i} {wl.shapes[i]}", si.weight(wl, i), wl.dtype, precision,
                          lr, kw)
        for t, (Wg, Mg, Og) in enumerate(traj[:steps]):
            G = grads[i][t] if grads is not None else si.grad(wl, i, t)
            errs = chk.check(G, Wg, Mg, Og)
            if report is not None:
                report.append((i, t) + errs)
            worst = _merge(worst, errs)
    _summary(wl.name, precision, worst)
    return worst


def run_lockstep(wl, steps, precision, watch, cfg=None, gpu_fill_others=False, oracle_kw=None,
                 dev=None, single_launch=None):
    """``steps`` Muon steps of the whole workload on the GPU; after each one, the oracle's
    step of every watched matrix from the oracle's own state, compared at once (nothing is
    kept but the oracle's state). Gradients of watched matrices come from the seeded CPU
    generator, once per step for both sides. Prints one line per step. Returns the worst
    errors as ``compare`` does. ``single_launch`` (True / False): after the compared steps,
    one more step with the library's launch counts on confirms that the plan runs its
    rounds as one persistent launch (or as one launch per product)."""
    dev = dev or torch.device("cuda", 0)
    watch = list(watch)
    kw = dict(oracle_kw or {})
    cfg = cfg or make_config(**{k: v for k, v in kw.items()
                                if k in ("lr", "beta", "nesterov", "ns_steps")})
    lr = kw.pop("lr", 0.02)
    W, M, O = _init_buffers(wl, watch, dev, gpu_fill_others, None)
    plan = MuonPlan(wl.shapes, [w.dtype for w in W], [w.dtype for w in W], precision, dev)
    checks = {i: StepChecker(f"matrix {i} {wl.shapes[i]}", si.weight(wl, i), wl.dtype,
                             precision, lr, kw) for i in watch}
    worst = [0.0, 0.0, 0.0, None]
    try:
        for t in range(steps):
            cpu_g = {i: si.grad(wl, i, t) for i in watch}
            G = [(cpu_g[i].to(dev) if i in cpu_g else
                  (gpu_fill_grad(wl, i, t, dev) if gpu_fill_others else si.grad(wl, i, t).to(dev)))
                 for i in range(wl.n)]
            plan.step(W, G, M, cfg, outs=O)
            torch.cuda.synchronize()
            del G
            step_worst = [0.0, 0.0, 0.0, None]
            for i in watch:
                errs = checks[i].check(cpu_g[i], f64(W[i]), f64(M[i]), f64(O[i]))
                step_worst = _merge(step_worst, errs)
            worst = _merge(worst, step_worst)
            es = "" if step_worst[3] is None else f" Wst {step_worst[3]:.2e}"
            print(f"[gpu] {wl.name} {precision} step {t + 1}/{steps}: O {step_worst[0]:.2e} "
                  f"W {step_worst[1]:.2e} M {step_worst[2]:.2e}{es}", flush=True)
        if single_launch is not None:
            plan.set_profiling(True)
            G = [si.grad(wl, i, 0).to(dev) for i in range(wl.n)]
            plan.step(W, G, M, cfg, outs=O)
            torch.cuda.synchronize()
            prof = plan.read_profile()
            assert (prof["rounds"][1] == 1) == single_launch, prof
            assert (prof["apply"][1] == 0) == single_launch, prof
    finally:
        plan.close()
    _summary(wl.name, precision, worst)
    return worst
