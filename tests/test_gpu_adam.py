"""GPU parity of the cautious-Adam entry point (muon_cautious_adam_step) with the fp64 CPU
oracle, through the C ABI.

Each step is checked element by element against the oracle's step from the same stored
state (the GPU's parameters and moments before the step, which both sides read exactly),
with a bound derived from fp32 arithmetic:

* m and v: 4 fp32 roundings of the magnitudes that enter them (beta1 |m| + (1-beta1) |g|,
  and beta2 v + (1-beta2) g^2);
* p: 2 roundings of |p|, plus lr times the error of the direction (the rounding of m carried
  through the bias correction and the denominator, and 16 roundings of |u|), plus the rounding
  of the decay term; half a bf16 unit (2^-8 |p|) more for a bf16 parameter, which is rounded
  once after the update;
* the mask: the direction has the sign of m, so fp32 can only take the other branch where
  |m| is within the rounding bound of m; there either branch's value is accepted.

Trajectories over several steps are also compared with the oracle run from the initial
values (relative Frobenius error <= 1e-5 for fp32 parameters, <= 3e-2 for bf16 ones).
"""
import numpy as np
import pytest
import torch

import oracle.cautious_adam as oa
import seeded_inputs as si
from orthogonalized_momentum_optimizer_amd import CautiousAdam, cautious_adam_step, make_adam_config

pytestmark = pytest.mark.gpu

E32 = 2.0 ** -24
TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def dev():
    return torch.device("cuda", 0)


def f64(t):
    return t.detach().double().cpu().numpy().reshape(-1)


def rel(x, y):
    d = np.linalg.norm(y)
    return float(np.linalg.norm(x - y) / d) if d > 0 else float(np.linalg.norm(x))


def check_step(prev, new, g, cfg, wd_mul, pdt, label, stats=None):
    """Element-wise check of one GPU step (new) against the oracle's step from the GPU's
    state before it (prev = (p, m, v)); all arrays float64 copies of stored values."""
    p0, m0, v0 = prev
    p1, m1, v1 = new
    t, lr, b1, b2, eps, wd = cfg.step, cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay
    lam = wd * wd_mul
    pr, mr, vr, mask = oa.cautious_adam_step(p0, g, m0, v0, t, lr, b1, b2, eps, wd, wd_mul)
    mag_m = b1 * np.abs(m0) + (1 - b1) * np.abs(g)
    mag_v = b2 * v0 + (1 - b2) * g * g
    assert np.all(np.abs(m1 - mr) <= 4 * E32 * mag_m), f"{label}: m differs"
    assert np.all(np.abs(v1 - vr) <= 4 * E32 * mag_v), f"{label}: v differs"
    bc1, bc2 = 1 - b1 ** t, 1 - b2 ** t
    with np.errstate(divide="ignore", invalid="ignore"):
        denom = np.sqrt(vr / bc2) + eps
        u = (mr / bc1) / denom
        du = 4 * E32 * mag_m / bc1 / denom + 16 * E32 * np.abs(u)
    tol = 2 * E32 * np.abs(pr) + lr * (du + 4 * E32 * abs(lam) * np.abs(p0)) + 1e-30
    if pdt == "bf16":
        tol = tol + 2.0 ** -8 * np.abs(pr)
    ok = np.abs(p1 - pr) <= tol
    ok |= np.isnan(p1) & np.isnan(pr)
    amb = np.abs(mr) <= 4 * E32 * mag_m
    if amb.any():
        other = np.where(mask, p0 - lr * u, p0 - lr * (u + lam * p0))
        ok |= amb & (np.abs(p1 - other) <= tol)
    bad = np.flatnonzero(~ok)
    assert bad.size == 0, (f"{label}: {bad.size} parameters differ, first at {bad[0]}: gpu "
                           f"{p1[bad[0]]!r} oracle {pr[bad[0]]!r} tol {tol[bad[0]]!r}")
    if stats is not None:
        stats["ambiguous"] = stats.get("ambiguous", 0) + int(amb.sum())
        stats["masked"] = stats.get("masked", 0) + int(mask.sum())
        stats["elements"] = stats.get("elements", 0) + mask.size
        err = np.abs(p1 - pr) / np.maximum(np.abs(pr), 1e-30)
        stats["worst_rel_p"] = max(stats.get("worst_rel_p", 0.0), float(np.max(err, initial=0)))


def make_state(aset, pdt="f32", gdt=None):
    gdt = gdt or pdt
    P = [si.adam_param(aset, i).to(TORCH_DT[pdt]).to(dev()).reshape(-1) for i in range(aset.n)]
    M = [torch.zeros(p.numel(), dtype=torch.float32, device=dev()) for p in P]
    V = [torch.zeros(p.numel(), dtype=torch.float32, device=dev()) for p in P]
    return P, M, V


def run_and_check(aset, steps, pdt, gdt, lr=1e-2, betas=(0.9, 0.99), eps=1e-8, wd=0.05,
                  t0=1, stats=None):
    P, M, V = make_state(aset, pdt, gdt)
    muls = [w for _, _, w in aset.tensors]
    traj = []
    for k in range(steps):
        G = [si.adam_grad(aset, i, k).to(TORCH_DT[gdt]).to(dev()).reshape(-1)
             for i in range(aset.n)]
        prev = [(f64(p), f64(m), f64(v)) for p, m, v in zip(P, M, V)]
        cfg = make_adam_config(lr, betas, eps, wd, t0 + k)
        cautious_adam_step(P, G, M, V, cfg, muls)
        torch.cuda.synchronize()
        for i in range(aset.n):
            check_step(prev[i], (f64(P[i]), f64(M[i]), f64(V[i])), f64(G[i]), cfg, muls[i], pdt,
                       f"{aset.name}[{aset.tensors[i][0]}] step {t0 + k}", stats)
        traj.append([f64(p) for p in P])
    return traj, cfg


@pytest.mark.parametrize("pdt,gdt", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32"),
                                     ("f32", "bf16")])
def test_adam_parity_ragged(pdt, gdt):
    aset = si.ADAM_SETS["ragged_small"]
    print(f"[adam] ragged_small p={pdt} g={gdt}", flush=True)
    stats = {}
    traj, cfg = run_and_check(aset, aset.steps, pdt, gdt, stats=stats)
    assert stats["masked"] > 1000 and stats["elements"] - stats["masked"] > 1000
    assert stats["ambiguous"] <= 1e-3 * stats["elements"]
    # trajectories against the oracle run from the initial stored values
    tol = 3e-2 if pdt == "bf16" else 1e-5
    for i in range(aset.n):
        p0 = si.adam_param(aset, i).to(TORCH_DT[pdt])
        gs = [si.adam_grad(aset, i, k).to(TORCH_DT[gdt]) for k in range(aset.steps)]
        ref = oa.cautious_adam_run(p0.reshape(-1), [g.reshape(-1) for g in gs], cfg.lr,
                                   cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay,
                                   aset.tensors[i][2])
        for k in range(aset.steps):
            e = rel(traj[k][i], ref[k][0])
            assert e <= tol, f"tensor {i} step {k}: trajectory rel err {e:.3e}"
    print(f"[adam] stats {stats}", flush=True)


def test_adam_edge_sizes_mixed_dtypes_shared_grad():
    """Empty, single-element, vector-tail and chunk-boundary sizes (4096 elements per block),
    all four dtype pairs in one call, and two tensors reading one gradient."""
    sizes = [0, 1, 7, 8, 9, 4095, 4096, 8193, 16389, 24576 + 3, 4097, 12288]
    dts = [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32"), ("f32", "bf16")]
    print("[adam] edge sizes", flush=True)
    r = si.rng(30, 2, 0, 0)
    P, G, M, V, muls, pd = [], [], [], [], [], []
    for j, n in enumerate(sizes):
        pdt, gdt = dts[j % 4]
        P.append(torch.tensor(r.normal(0, 0.5, n), dtype=TORCH_DT[pdt], device=dev()))
        G.append(torch.tensor(r.normal(0, 1.0, n), dtype=TORCH_DT[gdt], device=dev()))
        M.append(torch.tensor(r.normal(0, 0.1, n), dtype=torch.float32, device=dev()))
        V.append(torch.tensor(r.uniform(0, 0.1, n), dtype=torch.float32, device=dev()))
        muls.append([0.0, 1.0, 150.0][j % 3])
        pd.append(pdt)
    P.append(torch.tensor(r.normal(0, 0.5, 8193), dtype=torch.float32, device=dev()))
    G.append(G[7])                                   # shares tensor 7's gradient (8193, bf16)
    M.append(torch.zeros(8193, dtype=torch.float32, device=dev()))
    V.append(torch.zeros(8193, dtype=torch.float32, device=dev()))
    muls.append(150.0)
    pd.append("f32")
    cfg = make_adam_config(3e-3, (0.8, 0.95), 1e-10, 0.02, 7)
    prev = [(f64(p), f64(m), f64(v)) for p, m, v in zip(P, M, V)]
    cautious_adam_step(P, G, M, V, cfg, muls)
    torch.cuda.synchronize()
    for i in range(len(P)):
        check_step(prev[i], (f64(P[i]), f64(M[i]), f64(V[i])), f64(G[i]), cfg, muls[i], pd[i],
                   f"edge tensor {i} ({P[i].numel()} elements)")


def test_adam_many_tensors_several_launches():
    """70 tensors of one dtype pair: more than one launch's 32 pieces."""
    shapes = [((i * 977) % 5000 + 1,) for i in range(70)]
    aset = si.adam_custom([(s, [0.0, 1.0, 150.0][i % 3]) for i, s in enumerate(shapes)],
                          "bf16", steps=2, cfg_id=201)
    print("[adam] 70 tensors", flush=True)
    run_and_check(aset, 2, "bf16", "bf16", t0=3)


def test_adam_special_values():
    """Zero gradient with zero moments (no change, eps > 0); eps = 0 at step 1, where the
    direction is sign(g) exactly; a late step (bias corrections ~ 1); zero decay."""
    print("[adam] special values", flush=True)
    n = 10000
    r = si.rng(31, 2, 0, 0)
    p = torch.tensor(r.normal(0, 1, n), dtype=torch.float32, device=dev())
    z = torch.zeros(n, dtype=torch.float32, device=dev())
    m, v, p0 = z.clone(), z.clone(), p.clone()
    cautious_adam_step([p], [z], [m], [v], make_adam_config(0.1, (0.9, 0.999), 1e-8, 0.5, 1))
    torch.cuda.synchronize()
    assert torch.equal(p, p0) and not m.any() and not v.any()

    g = torch.tensor(r.normal(0, 1, n), dtype=torch.float32, device=dev())
    m.zero_(); v.zero_()
    cfg = make_adam_config(0.125, (0.9, 0.999), 0.0, 0.5, 1)
    cautious_adam_step([p], [g], [m], [v], cfg, [2.0])
    torch.cuda.synchronize()
    s = torch.sign(g)
    expect = p0 - 0.125 * (s + torch.where(s * p0 > 0, 1.0 * p0, torch.zeros_like(p0)))
    assert torch.allclose(p, expect, rtol=4 * E32, atol=1e-7)

    for t, wd in ((1_000_000, 0.1), (5, 0.0)):
        aset = si.adam_custom([((4099,), 150.0), ((129,), 1.0)], "f32", steps=2, cfg_id=202)
        run_and_check(aset, 2, "f32", "f32", wd=wd, t0=t)


def test_adam_matches_torch_adam_and_adamw_on_gpu():
    """Against PyTorch's own fp32 GPU Adam (decay 0) and AdamW (every element agreeing in
    sign, so the mask is all set), an implementation independent of the oracle."""
    print("[adam] torch Adam/AdamW", flush=True)
    n = 50000
    r = si.rng(32, 2, 0, 0)
    g0 = torch.tensor(r.normal(0, 1, n), dtype=torch.float32)
    p0 = torch.tensor(np.abs(r.normal(0, 1, n)), dtype=torch.float32) * torch.sign(g0)
    for wd, cls in ((0.0, torch.optim.Adam), (0.3, torch.optim.AdamW)):
        # the library's hyper-parameters are fp32: give torch the same (fp32-exact) values
        c = make_adam_config(1e-2, (0.9, 0.99), 1e-8, wd, 1)
        P = torch.nn.Parameter(p0.clone().to(dev()))
        opt = cls([P], lr=c.lr, betas=(c.beta1, c.beta2), eps=c.eps, weight_decay=c.weight_decay,
                  foreach=False)
        P.grad = g0.to(dev())
        opt.step()
        p, m, v = p0.clone().to(dev()), torch.zeros(n, device=dev()), torch.zeros(n, device=dev())
        cautious_adam_step([p], [g0.to(dev())], [m], [v], c)
        torch.cuda.synchronize()
        assert torch.allclose(p, P.detach(), rtol=1e-6, atol=1e-8), cls.__name__
        assert torch.allclose(m, opt.state[P]["exp_avg"], rtol=1e-6, atol=0)
        assert torch.allclose(v, opt.state[P]["exp_avg_sq"], rtol=1e-6, atol=0)


def test_adam_deterministic():
    aset = si.ADAM_SETS["ragged_small"]
    outs = []
    for _ in range(2):
        P, M, V = make_state(aset, "bf16", "bf16")
        G = [si.adam_grad(aset, i, 0).to(torch.bfloat16).to(dev()).reshape(-1)
             for i in range(aset.n)]
        cautious_adam_step(P, G, M, V, make_adam_config(1e-2, (0.9, 0.99), 1e-8, 0.05, 1),
                           [w for _, _, w in aset.tensors])
        torch.cuda.synchronize()
        outs.append([x.clone() for x in P + M + V])
    assert all(torch.equal(a, b) for a, b in zip(*outs))


def test_cautious_adam_optimizer_class():
    """The torch.optim front end: two groups (multipliers 150 and 0), 3 steps, any shapes."""
    print("[adam] CautiousAdam class", flush=True)
    r = si.rng(33, 2, 0, 0)
    shapes = [(300, 17), (5,), (2, 3, 129)]
    init = [r.normal(0, 0.5, s) for s in shapes]
    params = [torch.nn.Parameter(torch.tensor(x, dtype=torch.float32, device=dev()))
              for x in init]
    opt = CautiousAdam([{"params": params[:2], "wd_mul": 150.0},
                        {"params": params[2:], "wd_mul": 0.0}],
                       lr=1e-2, betas=(0.9, 0.99), eps=1e-8, weight_decay=1e-3)
    grads = [[r.normal(0, 1, s) for s in shapes] for _ in range(3)]
    for k in range(3):
        for p, g in zip(params, grads[k]):
            p.grad = torch.tensor(g, dtype=torch.float32, device=dev())
        opt.step()
    torch.cuda.synchronize()
    c = make_adam_config(1e-2, (0.9, 0.99), 1e-8, 1e-3, 1)    # fp32-rounded hyper-parameters
    for i, mul in enumerate([150.0, 150.0, 0.0]):
        ref = oa.cautious_adam_run(np.float32(init[i]), [np.float32(grads[k][i]) for k in range(3)],
                                   c.lr, c.beta1, c.beta2, c.eps, c.weight_decay, mul)
        assert rel(f64(params[i]), ref[-1][0].reshape(-1)) <= 1e-6


def _sampled_check(P, G, M, V, idx, cfg, muls, pdt, label, run):
    """Gathers the sampled elements before and after ``run`` and checks them."""
    prev = [(f64(P[i][ix]), f64(M[i][ix]), f64(V[i][ix]), f64(G[i][ix]))
            for i, ix in enumerate(idx)]
    run()
    torch.cuda.synchronize()
    for i, ix in enumerate(idx):
        p0, m0, v0, g = prev[i]
        check_step((p0, m0, v0), (f64(P[i][ix]), f64(M[i][ix]), f64(V[i][ix])), g, cfg, muls[i],
                   pdt, f"{label} tensor {i}")


def _sample_indices(n, r, k=50000, chunk=4096):
    ix = set(range(min(n, 4096))) | set(range(max(0, n - 4096), n))
    for c in range(chunk, n, max(chunk, (n // 64) // chunk * chunk)):
        ix |= set(range(max(0, c - 16), min(n, c + 16)))
    ix |= set(r.integers(0, n, size=min(k, n)).tolist())
    return torch.tensor(sorted(ix), dtype=torch.long, device=dev())


def test_adam_full_size_sampled():
    """The embedding-shaped set of a GPT-2-124M model (4 x 50257 x 768 bf16 + 64 scalars,
    one launch, as timed by the benchmark), three steps, sampled elements checked."""
    aset = si.ADAM_SETS["gpt2_124m_embed"]
    print(f"[adam] full size {aset.name} ({aset.elements()} elements)", flush=True)
    P, M, V = [], [], []
    gen = torch.Generator(device=dev())
    gen.manual_seed(aset.cfg_id)
    for i in range(aset.n):
        n = aset.numel(i)
        P.append((aset.param_std * torch.randn(n, generator=gen, device=dev())).to(torch.bfloat16))
        M.append(torch.zeros(n, dtype=torch.float32, device=dev()))
        V.append(torch.zeros(n, dtype=torch.float32, device=dev()))
    muls = [w for _, _, w in aset.tensors]
    r = si.rng(aset.cfg_id, 9, 0, 0)
    idx = [_sample_indices(p.numel(), r) for p in P]
    for t in range(1, 4):
        G = [(aset.grad_std * torch.randn(p.numel(), generator=gen, device=dev())).to(torch.bfloat16)
             for p in P]
        cfg = make_adam_config(1e-3, (0.9, 0.95), 1e-8, 0.01, t)
        _sampled_check(P, G, M, V, idx, cfg, muls, "bf16", f"full size step {t}",
                       lambda: cautious_adam_step(P, G, M, V, cfg, muls))


def test_adam_tensor_split_across_launches():
    """A bf16 tensor of 2^29 + 12345 elements is cut into two pieces (at most 2^29 elements
    per launch); elements around the cut and at the tail are checked."""
    n = (1 << 29) + 12345
    print(f"[adam] split tensor of {n} elements", flush=True)
    gen = torch.Generator(device=dev())
    gen.manual_seed(41)
    P = [(0.5 * torch.randn(n, generator=gen, device=dev())).to(torch.bfloat16)]
    G = [torch.randn(n, generator=gen, device=dev()).to(torch.bfloat16)]
    M = [0.1 * torch.randn(n, generator=gen, device=dev())]
    V = [0.1 * torch.rand(n, generator=gen, device=dev())]
    cut = 1 << 29
    ix = sorted(set(range(cut - 20000, cut + 12345)) | set(range(0, 9000)) |
                set(si.rng(41, 9, 0, 0).integers(0, n, size=50000).tolist()))
    idx = [torch.tensor(ix, dtype=torch.long, device=dev())]
    cfg = make_adam_config(1e-2, (0.9, 0.99), 1e-8, 0.1, 4)
    _sampled_check(P, G, M, V, idx, cfg, [150.0], "bf16", "split tensor",
                   lambda: cautious_adam_step(P, G, M, V, cfg, [150.0]))
    del P, G, M, V
    torch.cuda.empty_cache()
