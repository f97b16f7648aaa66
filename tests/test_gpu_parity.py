"""GPU parity: the HIP library through its C ABI against the CPU oracle, element by
element, on seeded inputs (run on an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from harness import TOL, compare, f64, rel, run_gpu
from orthogonalized_momentum_optimizer_amd import MuonPlan, make_config

pytestmark = pytest.mark.gpu

RAGGED = [(200, 328), (328, 200), (64, 64), (1, 37), (130, 1), (257, 129), (96, 160),
          (384, 128), (5, 3)]


def _announce(msg):
    print(f"[gpu] {msg}", flush=True)


@pytest.mark.parametrize("precision", ["bf16", "f32"])
def test_ragged_shapes_full_parity(precision):
    """Shapes spanning several 128-tiles with ragged tails, wide, tall, vectors and tiny."""
    _announce(f"ragged shapes {precision}")
    wl = si.custom(RAGGED, dtype="bf16", steps=3, cfg_id=101)
    gpu = run_gpu(wl, 3, precision)
    compare(wl, gpu, 3, precision)


@pytest.mark.parametrize("precision", ["bf16", "f32"])
def test_ragged_shapes_fp32_params(precision):
    _announce(f"ragged fp32 params {precision}")
    wl = si.custom([(100, 260), (260, 100), (33, 33)], dtype="f32", steps=2, cfg_id=102,
                   grad_std=1.0)
    gpu = run_gpu(wl, 2, precision)
    compare(wl, gpu, 2, precision)


@pytest.mark.parametrize("precision", ["bf16"])
def test_large_tile_products_ragged(precision):
    """Shape groups with mp >= 1024 use 256x256 tiles for the Gram and polynomial products:
    mp = 1152 leaves the last tile row half outside the matrix, 1024 is exactly four tiles,
    and the tall 1400x1030 runs transposed (mp 1152, np 1408)."""
    _announce(f"256-tile products {precision}")
    wl = si.custom([(1100, 1100), (1030, 1400), (1400, 1030), (1024, 1024), (1024, 1536)],
                   cfg_id=111, steps=2)
    gpu = run_gpu(wl, 2, precision)
    compare(wl, gpu, 2, precision)


def test_many_tiles_per_block_full_parity():
    """300 matrices of 128x384 (mp 128, np 384): 600 apply tiles, more than the device has
    compute units, so every persistent block walks several ragged tiles (each half outside
    its matrix); every element of every matrix is compared."""
    _announce("many tiles per block")
    wl = si.custom([(128, 384)] * 150 + [(384, 128)] * 150, cfg_id=112, steps=2)
    gpu = run_gpu(wl, 2, "bf16")
    compare(wl, gpu, 2, "bf16")


@pytest.mark.parametrize("precision", ["bf16", "f32"])
def test_gpt2_tiny_fp32_workload(precision):
    """64x256 fp32 matrix, one N(0,1) gradient reused for 3 steps."""
    _announce(f"gpt2_tiny_fp32 {precision}")
    wl = si.WORKLOADS["gpt2_tiny_fp32"]
    gpu = run_gpu(wl, wl.steps, precision)
    compare(wl, gpu, wl.steps, precision)
    # closed form with one reused gradient: W_3 = W_0 - 3 lr NS5(G/||G||)
    O_ref, _ = oracle.orthogonalize(f64(si.grad(wl, 0, 0)), 5)
    W3 = gpu[0][-1][0]
    W0 = f64(si.weight(wl, 0))
    assert rel(W0 - W3, 3 * 0.02 * O_ref) <= TOL[precision]




@pytest.mark.parametrize("precision", ["bf16", "f32"])
def test_tiny_fp32_fresh_gradient_each_step(precision):
    """The other reading of the 64x256 workload's text: a fresh N(0, 1) gradient every step
    instead of one reused (the closed form above no longer applies; oracle parity does)."""
    _announce(f"64x256 fp32, fresh gradient per step, {precision}")
    wl = si.custom([(64, 256)], dtype="f32", steps=3, grad_std=1.0, cfg_id=117)
    gpu = run_gpu(wl, 3, precision)
    compare(wl, gpu, 3, precision)


def test_iid_student_t_entries():
    """The other reading of the tall-stress workload's "heavy-tailed rows": every gradient
    entry i.i.d. 1e-3 * Student-t(3) (a few entries dominate the Frobenius norm), on two of
    its matrices of each orientation, 3 steps, against the oracle."""
    _announce("tall/wide 3072x768, i.i.d. Student-t(3) entries")
    wl = si.custom([(3072, 768), (768, 3072)] * 2, dtype="bf16", steps=3, cfg_id=118,
                   iid_t3_entries=True)
    gpu = run_gpu(wl, 3, "bf16", watch=[0, 1])
    compare(wl, gpu, 3, "bf16")






def test_gpt2_124m_share8_all_matrices():
    """One GPU's share at 8 GPUs (6 x 768x768 + 3 x 3072x768): few tiles per launch, every
    matrix compared over 3 steps."""
    wl = si.WORKLOADS["gpt2_124m_share8"]
    _announce("gpt2_124m_share8, all matrices")
    gpu = run_gpu(wl, 3, "bf16")
    compare(wl, gpu, 3, "bf16")


def test_groups_side_by_side_equal_group_by_group_bitwise():
    """A set too small to fill the device runs each phase over all shape groups at once; a
    larger one runs group by group. The same 9 matrices (6 x 768x768, 3 x 3072x768; 162
    apply tiles) alone and followed by 60 more 768x768 matrices (702 apply tiles) must give
    bitwise the same W, M and O."""
    _announce("side-by-side groups vs group by group")
    small = [(768, 768)] * 6 + [(3072, 768)] * 3
    a = run_gpu(si.custom(small, cfg_id=113, steps=2), 2, "bf16")
    b = run_gpu(si.custom(small + [(768, 768)] * 60, cfg_id=113, steps=2), 2, "bf16",
                watch=range(len(small)))
    for i in range(len(small)):
        for t in range(2):
            for x, y in zip(a[i][t], b[i][t]):
                assert np.array_equal(x, y), f"matrix {i} step {t}"


def test_more_groups_than_one_launch_holds():
    """Ten small shape groups (padded mp 128-512), too few tiles to fill the device, so they
    run side by side: the Gram and polynomial launches hold at most 8 groups (two launches
    here), apply takes the groups of each mp together. Every element is compared."""
    _announce("ten groups side by side")
    shapes = [(128, 128), (128, 256), (128, 384), (256, 256), (256, 512), (384, 384),
              (512, 128), (256, 384), (384, 512), (512, 512), (300, 40)]
    wl = si.custom(shapes, cfg_id=114, steps=2)
    gpu = run_gpu(wl, 2, "bf16")
    compare(wl, gpu, 2, "bf16")






def test_batch_equals_alone_bitwise():
    """A matrix's result does not depend on the other matrices of the call."""
    _announce("batch vs alone")
    wl = si.custom(RAGGED, dtype="bf16", steps=2, cfg_id=103)
    batch = run_gpu(wl, 2, "bf16")
    for i in (0, 1, 5, 7):
        one = si.custom([RAGGED[i]], dtype="bf16", steps=2, cfg_id=103)
        grads = [[si.grad(wl, i, t) for t in range(2)]]
        alone = run_gpu(one, 2, "bf16", grads=grads, W0=[si.weight(wl, i)])
        for t in range(2):
            for k in range(3):
                assert np.array_equal(batch[i][t][k], alone[0][t][k]), (i, t, k)


def test_apply_tile_sizes_agree_bitwise():
    """A set whose 256x256 apply tiles would leave at least half of the compute units idle
    runs 128x128 apply tiles instead. Both kernels add the same K slices in the same order,
    so a matrix gives bitwise the same W, M and O alone (9 tiles of 256: the 128-tile
    kernel) as inside a set of 20 (180 tiles of 256: the persistent 256-tile kernel); the
    tall and wide 384x1536 pair checks a wide group and the transposed path the same way."""
    _announce("apply 128 vs 256 tiles")
    for shapes, watch in (([(768, 768)] * 20, (0, 13, 19)),
                          ([(384, 1536), (1536, 384)] * 40, (0, 41, 79))):
        wl = si.custom(shapes, dtype="bf16", steps=2, cfg_id=116)
        batch = run_gpu(wl, 2, "bf16", watch=watch, gpu_fill_others=True)
        for i in watch:
            one = si.custom([shapes[i]], dtype="bf16", steps=2, cfg_id=116)
            grads = [[si.grad(wl, i, t) for t in range(2)]]
            alone = run_gpu(one, 2, "bf16", grads=grads, W0=[si.weight(wl, i)])
            for t in range(2):
                for k in range(3):
                    assert np.array_equal(batch[i][t][k], alone[0][t][k]), (shapes[i], i, t, k)
        compare(wl, {i: batch[i] for i in watch[:1]}, 2, "bf16")


def test_deterministic_bitwise():
    _announce("determinism")
    wl = si.custom([(384, 640), (640, 384), (200, 200)], dtype="bf16", steps=2, cfg_id=104)
    a = run_gpu(wl, 2, "bf16")
    b = run_gpu(wl, 2, "bf16")
    for i in a:
        for t in range(2):
            for k in range(3):
                assert np.array_equal(a[i][t][k], b[i][t][k])


def test_transpose_path_matches_wide_bitwise():
    """A tall matrix runs as its transpose: NS(G^T) equals NS(G)^T bit for bit."""
    _announce("transpose path")
    dev = torch.device("cuda", 0)
    G = si.grad(si.custom([(320, 192)], cfg_id=105), 0, 0).to(dev)
    outs = []
    for x in (G, G.t().contiguous()):
        plan = MuonPlan([x.shape], [torch.float32], [x.dtype], "bf16", dev)
        y = torch.empty(x.shape, dtype=torch.float32, device=dev)
        plan.newton_schulz([x], [y], make_config())
        torch.cuda.synchronize()
        outs.append(f64(y))
        plan.close()
    assert np.array_equal(outs[0], outs[1].T)


def test_step_on_transpose_is_transpose_bitwise():
    """A whole Muon step on (W^T, G^T) gives bitwise the transposes of W, M and O from the step
    on (W, G): momentum and update are elementwise, the wide form X0 and the sum of squares
    behind the norm are formed in the same order on both paths. Column counts cover the
    8-wide, the 4-wide and the per-element access paths."""
    _announce("step on the transpose")
    dev = torch.device("cuda", 0)
    for r, c in ((320, 192), (200, 68), (130, 37)):
        wl = si.custom([(r, c)], dtype="bf16", steps=2, cfg_id=119)
        W0, grads = si.weight(wl, 0), [si.grad(wl, 0, t) for t in range(2)]
        res = []
        for tr in (False, True):
            f = (lambda x: x.t().contiguous()) if tr else (lambda x: x)
            W = f(W0).to(dev)
            M = torch.zeros(W.shape, dtype=torch.float32, device=dev)
            O = torch.empty(W.shape, dtype=torch.float32, device=dev)
            plan = MuonPlan([W.shape], [W.dtype], [W.dtype], "bf16", dev)
            for t in range(2):
                plan.step([W], [f(grads[t]).to(dev)], [M], make_config(), outs=[O])
            torch.cuda.synchronize()
            plan.close()
            res.append([f64(x) for x in (W, M, O)])
        for a, b in zip(res[0], res[1]):
            assert np.array_equal(a, b.T), (r, c)


def test_newton_schulz_entry_against_oracle():
    _announce("newton_schulz entry")
    dev = torch.device("cuda", 0)
    wl = si.custom([(256, 512), (512, 256), (100, 100)], cfg_id=106)
    for prec, odt in (("bf16", torch.bfloat16), ("f32", torch.float32)):
        X = [si.grad(wl, i, 0).to(dev) for i in range(wl.n)]
        Y = [torch.empty(s, dtype=odt, device=dev) for s in wl.shapes]
        plan = MuonPlan(wl.shapes, [odt] * wl.n, [x.dtype for x in X], prec, dev)
        plan.newton_schulz(X, Y, make_config(ns_steps=5))
        torch.cuda.synchronize()
        plan.close()
        for i in range(wl.n):
            ref, _ = oracle.orthogonalize(f64(X[i].cpu()), 5)
            e = rel(f64(Y[i]), ref)
            tol = TOL[prec] if odt == torch.float32 else TOL["bf16"]
            assert e <= tol, (prec, i, e)


def test_zero_padding_exact():
    """A 700x700 matrix and the same matrix zero-padded to 768x768 give identical results
    on the shared block and exact zeros elsewhere."""
    _announce("padding")
    dev = torch.device("cuda", 0)
    G = si.grad(si.custom([(700, 700)], cfg_id=107), 0, 0).to(dev)
    P = torch.zeros(768, 768, dtype=G.dtype, device=dev)
    P[:700, :700] = G
    ys = []
    for x in (G, P):
        plan = MuonPlan([x.shape], [torch.float32], [x.dtype], "bf16", dev)
        y = torch.empty(x.shape, dtype=torch.float32, device=dev)
        plan.newton_schulz([x], [y], make_config())
        torch.cuda.synchronize()
        plan.close()
        ys.append(f64(y))
    assert np.array_equal(ys[1][:700, :700], ys[0])
    assert not ys[1][700:, :].any() and not ys[1][:, 700:].any()


@pytest.mark.parametrize("precision", ["bf16", "f32"])
def test_ns_steps_zero_and_one(precision):
    _announce(f"ns_steps 0/1 {precision}")
    wl = si.custom([(96, 200), (200, 96)], cfg_id=108, steps=2)
    for k in (0, 1):
        gpu = run_gpu(wl, 2, precision, cfg=make_config(ns_steps=k))
        compare(wl, gpu, 2, precision, oracle_kw=dict(ns_steps=k))


# A cascade of per-round quintics: three rounds of the fixed map, then two rounds of the
# textbook quintic Newton-Schulz map p(x) = (15x - 10x^3 + 3x^5) / 8, which fixes 1 with
# zero slope and so polishes the band the fixed map leaves.
SCHEDULE = [(3.4445, -4.7750, 2.0315)] * 3 + [(1.875, -1.25, 0.375)] * 2


@pytest.mark.parametrize("precision", ["bf16", "f32"])
def test_coefficient_schedule(precision):
    _announce(f"coefficient schedule {precision}")
    wl = si.custom([(96, 200), (200, 96), (256, 256)], cfg_id=110, steps=2)
    gpu = run_gpu(wl, 2, precision, cfg=make_config(schedule=SCHEDULE))
    compare(wl, gpu, 2, precision, oracle_kw=dict(schedule=SCHEDULE))


def test_coefficient_schedule_polishes_singular_values():
    """With the polishing rounds the bf16 result's singular values sit much closer to 1
    than with the fixed map alone (a property of the method, checked on the GPU output)."""
    _announce("schedule polish")
    dev = torch.device("cuda", 0)
    g = torch.Generator(device="cpu").manual_seed(5)
    x = torch.randn(256, 512, generator=g).to(torch.bfloat16).to(dev)
    spreads = []
    for cfg in (make_config(), make_config(schedule=SCHEDULE)):
        y = torch.empty(256, 512, dtype=torch.float32, device=dev)
        plan = MuonPlan([(256, 512)], [torch.float32], [torch.bfloat16], "bf16", dev)
        plan.newton_schulz([x], [y], cfg)
        torch.cuda.synchronize()
        plan.close()
        sv = np.linalg.svd(f64(y), compute_uv=False)
        spreads.append(float(np.max(np.abs(sv - 1.0))))
    assert spreads[0] > 0.15 and spreads[1] < 0.5 * spreads[0], spreads


@pytest.mark.parametrize("precision", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [1e-22, 1e22])
@pytest.mark.parametrize("eps", [1e-7, 0.0])
def test_extreme_gradient_scales(precision, scale, eps):
    """Gradients whose entries sit near 1e-25 or 1e19 (N(0, 1e-3) draws times the scale,
    stored in bf16). Squares of the small ones underflow fp32 and sums of squares of the
    large ones overflow it, so the norm is summed in double and X0 is rescaled by a power of
    two before the first Gram product. With eps = 0 the normalisation is exact, with the
    default eps the small set is dominated by eps (O = p^5 applied to U / eps)."""
    _announce(f"gradient scale {scale:g}, eps {eps:g}, {precision}")
    wl = si.custom([(200, 328), (328, 200), (256, 256)], dtype="bf16", steps=2, cfg_id=120)
    grads = [[(si.grad(wl, i, t).float() * scale).to(torch.bfloat16) for t in range(2)]
             for i in range(wl.n)]
    for g in grads:
        assert all(torch.isfinite(x.float()).all() and x.float().abs().max() > 0 for x in g)
    gpu = run_gpu(wl, 2, precision, cfg=make_config(eps=eps), grads=grads)
    compare(wl, gpu, 2, precision, grads=grads, oracle_kw=dict(eps=eps))


def test_non_nesterov_and_other_hyperparameters():
    _announce("hyper-parameters")
    wl = si.custom([(128, 384)], cfg_id=109, steps=3)
    kw = dict(lr=0.05, beta=0.9, nesterov=False)
    gpu = run_gpu(wl, 3, "bf16", cfg=make_config(**kw))
    compare(wl, gpu, 3, "bf16", oracle_kw=kw)


def test_zero_gradient_leaves_weights():
    _announce("zero gradient")
    wl = si.custom([(128, 256), (300, 100)], cfg_id=110, steps=1)
    grads = [[torch.zeros(s, dtype=torch.bfloat16)] for s in wl.shapes]
    gpu = run_gpu(wl, 1, "bf16", grads=grads)
    for i in range(wl.n):
        W, M, O = gpu[i][0]
        assert not O.any() and not M.any()
        assert np.array_equal(W, f64(si.weight(wl, i)))


def test_nan_stays_in_its_matrix():
    _announce("NaN isolation")
    wl = si.custom([(128, 256), (128, 256), (256, 128)], cfg_id=111, steps=1)
    clean = [[si.grad(wl, i, 0)] for i in range(wl.n)]
    dirty = [[g[0].clone()] for g in clean]
    dirty[1][0][5, 7] = float("nan")
    a = run_gpu(wl, 1, "bf16", grads=clean)
    b = run_gpu(wl, 1, "bf16", grads=dirty)
    assert np.isnan(b[1][0][2]).any()
    for i in (0, 2):
        for k in range(3):
            assert np.array_equal(a[i][0][k], b[i][0][k])


def test_resume_bitwise():
    """4 steps equal 2 steps, a copy of (W, M) into fresh buffers, and 2 more steps."""
    _announce("resume")
    dev = torch.device("cuda", 0)
    wl = si.custom([(192, 320), (320, 192)], cfg_id=112, steps=4)
    cfg = make_config()

    def fresh():
        W = [si.weight(wl, i).to(dev) for i in range(wl.n)]
        M = [torch.zeros(s, dtype=torch.float32, device=dev) for s in wl.shapes]
        return W, M

    plan = MuonPlan(wl.shapes, [torch.bfloat16] * wl.n, [torch.bfloat16] * wl.n, "bf16", dev)
    W, M = fresh()
    for t in range(4):
        plan.step(W, [si.grad(wl, i, t).to(dev) for i in range(wl.n)], M, cfg)
    W2, M2 = fresh()
    for t in range(2):
        plan.step(W2, [si.grad(wl, i, t).to(dev) for i in range(wl.n)], M2, cfg)
    torch.cuda.synchronize()
    W3 = [w.cpu().to(dev) for w in W2]
    M3 = [m.cpu().to(dev) for m in M2]
    for t in range(2, 4):
        plan.step(W3, [si.grad(wl, i, t).to(dev) for i in range(wl.n)], M3, cfg)
    torch.cuda.synchronize()
    plan.close()
    for i in range(wl.n):
        assert torch.equal(W[i], W3[i]) and torch.equal(M[i], M3[i])


def test_output_band_of_quintic():
    """Singular values of the GPU result follow p^5 of the normalised input singular values
    within bf16 error, and stay inside the band of the 5-fold map."""
    _announce("band")
    dev = torch.device("cuda", 0)
    for k, shp in enumerate([(64, 256), (256, 768)]):
        x = si.grad(si.custom([shp], cfg_id=113 + k), 0, 0).to(dev)
        plan = MuonPlan([shp], [torch.float32], [x.dtype], "bf16", dev)
        y = torch.empty(shp, dtype=torch.float32, device=dev)
        plan.newton_schulz([x], [y], make_config())
        torch.cuda.synchronize()
        plan.close()
        xs = f64(x)
        s_in = np.sort(np.linalg.svd(xs, compute_uv=False) / np.linalg.norm(xs))
        s_out = np.sort(np.linalg.svd(f64(y), compute_uv=False))
        a, b, c = oracle.DEFAULT_ABC
        s5 = s_in.copy()
        for _ in range(5):
            s5 = a * s5 + b * s5 ** 3 + c * s5 ** 5
        assert np.max(np.abs(np.sort(s5) - s_out)) < 0.05
        assert s_out.max() < 1.202369 + 0.05 and s_out.min() > 0.681831 - 0.05
