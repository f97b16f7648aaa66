"""Host-side tests of the C ABI: exported symbols, defaults, plan layout and argument
validation. Validation errors are raised before any HIP call, so these run without a GPU.
Calls that pass fake device addresses run only where no GPU is present; the gpu-marked
variants at the end repeat the checks with real buffers."""
import ctypes
import os
import re

import pytest
import torch

from orthogonalized_momentum_optimizer_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
HEADERS = sorted(os.path.join(INCLUDE, h) for h in os.listdir(INCLUDE) if h.endswith(".h"))

no_gpu_only = pytest.mark.skipif(torch.cuda.is_available(),
                                 reason="fake device addresses are only used without a GPU")


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(muon_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = L.lib()
    names = declared_functions()
    assert len(names) >= 12 and "muon_cautious_adam_step" in names
    for name in names:
        assert hasattr(lib, name), f"{name} is declared in include/ but not exported"
    assert sorted(L.EXPORTED) == names


def test_single_hip_runtime_in_process():
    L.lib()
    maps = [ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln]
    assert len(set(maps)) == 1, set(maps)


def test_config_default():
    c = L.muon_config_default()
    assert (round(c.lr, 6), round(c.beta, 6), c.nesterov, c.ns_steps) == (0.02, 0.95, 1, 5)
    assert (round(c.a, 4), round(c.b, 4), round(c.c, 4)) == (3.4445, -4.775, 2.0315)
    assert abs(c.eps - 1e-7) < 1e-12
    assert c.row_equalize == 0 and abs(c.row_beta - 0.95) < 1e-7 and abs(c.row_eps - 1e-8) < 1e-15


def test_status_strings():
    for code, name in [(0, "MUON_OK"), (-1, "MUON_ERR_INVALID_ARG"), (-2, "MUON_ERR_UNSUPPORTED"),
                       (-3, "MUON_ERR_WORKSPACE"), (-4, "MUON_ERR_HIP")]:
        assert L.muon_status_string(code) == name


def _ws_expected(shapes, esz):
    """Workspace layout: per padded wide group X0, X1 (count*mp*np), A, B (count*mp*mp),
    partial sums (count * 64x64 tiles of X, doubles), scales (16 B per matrix), partial row sums and
    row factors of the row equaliser (count*8*np and count*np floats), each 256-aligned; then
    the single-launch rounds' queues, flag and completion counters (8 x 16 + 16 words and 3 x 16
    rounds x count words per group, 4 bytes each)."""
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    groups = {}
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        key = ((m + 127) // 128 * 128, (n + 127) // 128 * 128)
        groups[key] = groups.get(key, 0) + 1
    tot = 0
    for (mp, np_), cnt in groups.items():
        tot = al(tot + cnt * mp * np_ * esz)
        tot = al(tot + cnt * mp * np_ * esz)
        tot = al(tot + cnt * mp * mp * esz)
        tot = al(tot + cnt * mp * mp * esz)
        tot = al(tot + cnt * (mp // 64) * (np_ // 64) * 8)
        tot = al(tot + cnt * 16)
        tot = al(tot + cnt * 8 * np_ * 4)
        tot = al(tot + cnt * np_ * 4)
    if groups:
        tot = al(tot + 4 * (8 * 16 + 16 + sum(3 * 16 * cnt for cnt in groups.values())))
    return tot


@pytest.mark.parametrize("prec,esz", [(L.MUON_NS_BF16, 2), (L.MUON_NS_F32_DEBUG, 4)])
def test_plan_workspace_layout(prec, esz):
    shapes = [(768, 768)] * 4 + [(3072, 768), (768, 3072)] + [(700, 650), (5, 3)]
    p = L.muon_plan_create([s[0] for s in shapes], [s[1] for s in shapes],
                           [0] * len(shapes), [0] * len(shapes), prec)
    try:
        assert L.muon_plan_workspace_size(p) == _ws_expected(shapes, esz)
    finally:
        L.muon_plan_destroy(p)


def test_empty_plan():
    p = L.muon_plan_create([], [], [], [])
    assert L.muon_plan_workspace_size(p) == 0
    L.muon_step(p, None, 0, L.muon_config_default(), 0, 0, 0)   # n = 0 is a no-op
    L.muon_plan_destroy(p)


@pytest.mark.parametrize("rows,cols,pdt,gdt,code", [
    ([0], [4], [0], [0], L.MUON_ERR_INVALID_ARG),
    ([4], [-1], [0], [0], L.MUON_ERR_INVALID_ARG),
    ([40000], [4], [0], [0], L.MUON_ERR_UNSUPPORTED),
    ([20000], [20000], [0], [0], L.MUON_ERR_UNSUPPORTED),
    ([4], [4], [7], [0], L.MUON_ERR_INVALID_ARG),
    ([4], [4], [0], [2], L.MUON_ERR_INVALID_ARG),
])
def test_plan_create_rejects(rows, cols, pdt, gdt, code):
    with pytest.raises(L.MuonError) as e:
        L.muon_plan_create(rows, cols, pdt, gdt)
    assert e.value.status == code
    assert L.muon_last_error()


def test_plan_create_rejects_bad_precision():
    with pytest.raises(L.MuonError) as e:
        L.muon_plan_create([4], [4], [0], [0], 5)
    assert e.value.status == L.MUON_ERR_INVALID_ARG


def test_set_concurrency_validates_its_arguments():
    p = L.muon_plan_create([8, 300], [8, 600], [0, 0], [0, 0])   # two shape groups
    for bad in (0, -1, L.MUON_MAX_STREAMS + 1):
        with pytest.raises(L.MuonError) as e:
            L.muon_plan_set_concurrency(p, bad)
        assert e.value.status == L.MUON_ERR_INVALID_ARG
        assert "streams" in L.muon_last_error()
    L.muon_plan_set_concurrency(p, 1)   # sequential: makes no HIP call
    L.muon_plan_destroy(p)
    assert L.lib().muon_plan_set_concurrency(None, 2) == L.MUON_ERR_INVALID_ARG


def test_profile_calls_on_plan():
    p = L.muon_plan_create([8], [8], [0], [0])
    prof = L.muon_plan_read_profile(p)
    assert set(prof) == set(L.KERNEL_KINDS) and all(v == (0.0, 0) for v in prof.values())
    L.muon_plan_destroy(p)


# ---- validation of muon_step / muon_newton_schulz, with fake addresses ---------------------

BASE = 1 << 40   # a fake, 4 KiB aligned device address range; never dereferenced


def _fake_call(mutate=None, cfg_mut=None, ws_off=0, ws_bytes=None, n=None):
    shapes = [(64, 128), (128, 64)]
    p = L.muon_plan_create([s[0] for s in shapes], [s[1] for s in shapes], [0, 0], [0, 0])
    ws = L.muon_plan_workspace_size(p)
    ents = []
    addr = BASE
    for r, c in shapes:
        e = [addr, addr + (1 << 20), addr + (2 << 20), 0, r, c, 0, 0, addr + (3 << 20)]
        addr += 4 << 20
        ents.append(e)
    if mutate:
        mutate(ents)
    mats = L.make_matrices([tuple(e) for e in ents])
    cfg = L.muon_config_default()
    if cfg_mut:
        cfg_mut(cfg)
    wsp = BASE + (64 << 20) + ws_off
    try:
        with pytest.raises(L.MuonError) as e:
            L.muon_step(p, mats, len(shapes) if n is None else n, cfg, wsp,
                        ws if ws_bytes is None else ws_bytes, 0)
        return e.value.status, L.muon_last_error()
    finally:
        L.muon_plan_destroy(p)


@no_gpu_only
@pytest.mark.parametrize("case,code", [
    ("null_param", L.MUON_ERR_INVALID_ARG),
    ("null_grad", L.MUON_ERR_INVALID_ARG),
    ("null_momentum", L.MUON_ERR_INVALID_ARG),
    ("misaligned_grad", L.MUON_ERR_INVALID_ARG),
    ("misaligned_out", L.MUON_ERR_INVALID_ARG),
    ("shape_mismatch", L.MUON_ERR_INVALID_ARG),
    ("dtype_mismatch", L.MUON_ERR_INVALID_ARG),
    ("param_overlaps_grad", L.MUON_ERR_INVALID_ARG),
    ("momentum_overlaps_other_param", L.MUON_ERR_INVALID_ARG),
    ("out_overlaps_grad", L.MUON_ERR_INVALID_ARG),
])
def test_step_rejects_matrices(case, code):
    def mutate(e):
        if case == "null_param": e[0][0] = 0
        if case == "null_grad": e[0][1] = 0
        if case == "null_momentum": e[1][2] = 0
        if case == "misaligned_grad": e[1][1] += 8
        if case == "misaligned_out": e[0][3] = BASE + (3 << 20) + 4
        if case == "shape_mismatch": e[1][4] = 65
        if case == "dtype_mismatch": e[0][6] = 1
        if case == "param_overlaps_grad": e[0][1] = e[0][0] + 64
        if case == "momentum_overlaps_other_param": e[1][2] = e[0][0]
        if case == "out_overlaps_grad": e[0][3] = e[1][1]
    status, msg = _fake_call(mutate)
    assert status == code and msg


@no_gpu_only
def test_step_allows_shared_read_only_gradient():
    """Two matrices may read the same gradient buffer; the call then passes validation and
    fails only when it tries to launch (there is no GPU here)."""
    def mutate(e):
        e[1][1] = e[0][1]
        e[1][4], e[1][5] = 128, 64
    status, msg = _fake_call(mutate)
    assert status == L.MUON_ERR_HIP, msg


@no_gpu_only
@pytest.mark.parametrize("field,value", [("ns_steps", -1), ("ns_steps", 65), ("eps", -1.0),
                                         ("a", float("nan")), ("lr", float("inf")),
                                         ("beta", float("nan"))])
def test_step_rejects_config(field, value):
    status, _ = _fake_call(cfg_mut=lambda c: setattr(c, field, value))
    assert status == L.MUON_ERR_INVALID_ARG


@no_gpu_only
def test_step_rejects_non_finite_schedule():
    from orthogonalized_momentum_optimizer_amd import make_config
    good = make_config(ns_steps=2, schedule=[(3.4445, -4.775, 2.0315), (1.875, -1.25, 0.375)])
    bad = make_config(ns_steps=2, schedule=[(3.4445, -4.775, 2.0315), (1.875, float("nan"), 0.375)])
    status, msg = _fake_call(cfg_mut=lambda c: setattr(c, "schedule", bad.schedule))
    assert status == L.MUON_ERR_INVALID_ARG and "schedule" in msg
    status, msg = _fake_call(cfg_mut=lambda c: (setattr(c, "schedule", good.schedule),
                                                setattr(c, "ns_steps", 2)))
    assert status == L.MUON_ERR_HIP, msg     # passes validation, fails only at launch


def test_make_config_schedule_length():
    from orthogonalized_momentum_optimizer_amd import make_config
    with pytest.raises(ValueError):
        make_config(ns_steps=3, schedule=[(1.0, 0.0, 0.0)] * 2)
    cfg = make_config(ns_steps=2, schedule=[(1.0, 2.0, 3.0), (4.0, 5.0, 6.0)])
    assert [cfg.schedule[k] for k in range(6)] == [1.0, 2.0, 3.0, 4.0, 5.0, 6.0]
    assert not make_config().schedule


@no_gpu_only
@pytest.mark.parametrize("case", ["null_row_var", "misaligned_row_var", "row_var_overlaps_param",
                                  "row_var_overlaps_other_row_var", "bad_row_beta",
                                  "negative_row_eps", "nan_row_eps", "row_equalize_2"])
def test_step_rejects_row_equaliser_arguments(case):
    def mutate(e):
        if case == "null_row_var": e[1][8] = 0
        if case == "misaligned_row_var": e[0][8] += 4
        if case == "row_var_overlaps_param": e[0][8] = e[0][0] + 16
        if case == "row_var_overlaps_other_row_var": e[1][8] = e[0][8] + 128
    def cfg_mut(c):
        c.row_equalize = 2 if case == "row_equalize_2" else 1
        if case == "bad_row_beta": c.row_beta = 1.0
        if case == "negative_row_eps": c.row_eps = -1.0
        if case == "nan_row_eps": c.row_eps = float("nan")
    status, msg = _fake_call(mutate, cfg_mut)
    assert status == L.MUON_ERR_INVALID_ARG and msg


@no_gpu_only
def test_row_state_checked_only_when_equalising():
    """Without row_equalize a NULL or overlapping row_var is ignored (the call then fails only
    at launch, there is no GPU here); with it, a valid set passes validation too."""
    def mutate(e):
        e[0][8] = 0
        e[1][8] = e[1][0]
    assert _fake_call(mutate)[0] == L.MUON_ERR_HIP
    status, msg = _fake_call(cfg_mut=lambda c: setattr(c, "row_equalize", 1))
    assert status == L.MUON_ERR_HIP, msg


@no_gpu_only
def test_step_rejects_workspace():
    assert _fake_call(ws_off=16)[0] == L.MUON_ERR_WORKSPACE
    assert _fake_call(ws_bytes=1024)[0] == L.MUON_ERR_WORKSPACE
    status, msg = _fake_call(mutate=lambda e: e[0].__setitem__(0, BASE + (64 << 20)))
    assert status == L.MUON_ERR_INVALID_ARG, msg          # param inside the workspace
    assert _fake_call(n=1)[0] == L.MUON_ERR_INVALID_ARG   # n differs from the plan


@no_gpu_only
def test_newton_schulz_rejects():
    p = L.muon_plan_create([64], [96], [0], [0])
    ws = L.muon_plan_workspace_size(p)
    cfg = L.muon_config_default()
    wsp = BASE + (64 << 20)
    cases = [([0], [BASE]), ([BASE + 8], [BASE + (1 << 20)]), ([BASE], [BASE + 64])]
    for ins, outs in cases:
        with pytest.raises(L.MuonError) as e:
            L.muon_newton_schulz(p, ins, outs, cfg, wsp, ws, 0)
        assert e.value.status == L.MUON_ERR_INVALID_ARG
    L.muon_plan_destroy(p)


# ---- the same validation with real buffers, on the GPU --------------------------------------

@pytest.mark.gpu
def test_step_rejects_with_real_buffers():
    from orthogonalized_momentum_optimizer_amd import MuonPlan, make_config
    dev = torch.device("cuda", 0)
    plan = MuonPlan([(64, 128)], [torch.bfloat16], [torch.bfloat16], "bf16", dev)
    W = torch.zeros(64, 128, dtype=torch.bfloat16, device=dev)
    G = torch.zeros(64, 128, dtype=torch.bfloat16, device=dev)
    M = torch.zeros(64, 128, dtype=torch.float32, device=dev)
    big = torch.zeros(2 * 64 * 128, dtype=torch.float32, device=dev)
    cfg = make_config()
    with pytest.raises(L.MuonError) as e:       # momentum 4 bytes off a 16-byte boundary
        plan.step([W], [G], [big[1:1 + 64 * 128].view(64, 128)], cfg)
    assert e.value.status == L.MUON_ERR_INVALID_ARG
    with pytest.raises(L.MuonError) as e:       # update_out overlapping the momentum buffer
        plan.step([W], [G], [M], cfg, outs=[M])
    assert e.value.status == L.MUON_ERR_INVALID_ARG
    with pytest.raises(L.MuonError):
        cfg.ns_steps = 65
        plan.step([W], [G], [M], cfg)
    cfg.ns_steps = 5
    ws = plan.workspace
    with pytest.raises(L.MuonError) as e:
        L.muon_step(plan.handle, plan._matrices([W], [G], [M], None), 1, cfg,
                    ws.data_ptr(), plan.ws_bytes - 256, torch.cuda.current_stream().cuda_stream)
    assert e.value.status == L.MUON_ERR_WORKSPACE
    plan.step([W], [G], [M], cfg)    # valid call still works afterwards
    torch.cuda.synchronize()
    plan.close()


# ---- cautious Adam: defaults and validation ---------------------------------------------------

def test_adam_config_default():
    c = L.muon_adam_config_default()
    assert (round(c.lr, 9), round(c.beta1, 6), round(c.beta2, 6)) == (1e-3, 0.9, 0.999)
    assert abs(c.eps - 1e-8) < 1e-15 and c.weight_decay == 0.0 and c.step == 1


def test_adam_empty_call_is_a_no_op():
    L.muon_cautious_adam_step(None, 0, L.muon_adam_config_default(), 0)


def _adam_fake_call(mutate=None, cfg_mut=None, n=None):
    ents = []
    addr = BASE
    for numel, pdt in ((1000, 0), (37, 1)):
        ents.append([addr, addr + (1 << 20), addr + (2 << 20), addr + (3 << 20), numel, pdt, 0,
                     1.0])
        addr += 4 << 20
    if mutate:
        mutate(ents)
    arr = L.make_adam_tensors([tuple(e) for e in ents])
    cfg = L.muon_adam_config_default()
    if cfg_mut:
        cfg_mut(cfg)
    with pytest.raises(L.MuonError) as e:
        L.muon_cautious_adam_step(arr, len(ents) if n is None else n, cfg, 0)
    return e.value.status, L.muon_last_error()


@no_gpu_only
@pytest.mark.parametrize("case,code", [
    ("null_param", L.MUON_ERR_INVALID_ARG),
    ("null_exp_avg_sq", L.MUON_ERR_INVALID_ARG),
    ("misaligned_grad", L.MUON_ERR_INVALID_ARG),
    ("negative_numel", L.MUON_ERR_INVALID_ARG),
    ("huge_numel", L.MUON_ERR_UNSUPPORTED),
    ("bad_dtype", L.MUON_ERR_INVALID_ARG),
    ("nan_wd_mul", L.MUON_ERR_INVALID_ARG),
    ("param_overlaps_grad", L.MUON_ERR_INVALID_ARG),
    ("exp_avg_overlaps_other_param", L.MUON_ERR_INVALID_ARG),
    ("moments_alias", L.MUON_ERR_INVALID_ARG),
    ("negative_n", L.MUON_ERR_INVALID_ARG),
])
def test_adam_rejects_tensors(case, code):
    def mutate(e):
        if case == "null_param": e[0][0] = 0
        if case == "null_exp_avg_sq": e[1][3] = 0
        if case == "misaligned_grad": e[1][1] += 4
        if case == "negative_numel": e[0][4] = -1
        if case == "huge_numel": e[0][4] = (1 << 40) + 1
        if case == "bad_dtype": e[1][6] = 3
        if case == "nan_wd_mul": e[0][7] = float("nan")
        if case == "param_overlaps_grad": e[0][1] = e[0][0] + 16
        if case == "exp_avg_overlaps_other_param": e[1][2] = e[0][0] + 32
        if case == "moments_alias": e[0][3] = e[0][2]
    status, msg = _adam_fake_call(mutate, n=-1 if case == "negative_n" else None)
    assert status == code and msg


@no_gpu_only
@pytest.mark.parametrize("field,value", [("lr", float("nan")), ("eps", -1e-8),
                                         ("eps", float("inf")), ("beta1", 1.0),
                                         ("beta2", -0.1), ("beta1", float("nan")),
                                         ("weight_decay", float("inf")), ("step", 0)])
def test_adam_rejects_config(field, value):
    status, msg = _adam_fake_call(cfg_mut=lambda c: setattr(c, field, value))
    assert status == L.MUON_ERR_INVALID_ARG and msg


@no_gpu_only
def test_adam_decay_overflow_rejected():
    def mutate(e):
        e[0][7] = 3e38
    status, msg = _adam_fake_call(mutate, cfg_mut=lambda c: setattr(c, "weight_decay", 10.0))
    assert status == L.MUON_ERR_INVALID_ARG and "overflows" in msg


@no_gpu_only
def test_adam_validation_passes_for_legal_sets():
    """Empty tensors may carry NULL pointers, and tensors may share one read-only gradient:
    such calls pass validation and fail only when they launch (there is no GPU here)."""
    def mutate(e):
        e[1][1] = e[0][1]
        e.append([0, 0, 0, 0, 0, 0, 0, 1.0])
    status, msg = _adam_fake_call(mutate)
    assert status == L.MUON_ERR_HIP, msg


# ---- randomized plans: grouping and workspace size against a model of the layout -----------

from hypothesis import given, settings, strategies as st  # noqa: E402


@settings(max_examples=60, deadline=None)
@given(st.lists(st.tuples(st.integers(1, 3000), st.integers(1, 3000),
                          st.sampled_from([0, 1]), st.sampled_from([0, 1])),
                min_size=1, max_size=12),
       st.sampled_from([(L.MUON_NS_BF16, 2), (L.MUON_NS_F32_DEBUG, 4)]))
def test_random_plans_workspace_model(mats, prec_esz):
    prec, esz = prec_esz
    rows, cols = [m[0] for m in mats], [m[1] for m in mats]
    p = L.muon_plan_create(rows, cols, [m[2] for m in mats], [m[3] for m in mats], prec)
    try:
        assert L.muon_plan_workspace_size(p) == _ws_expected(list(zip(rows, cols)), esz)
    finally:
        L.muon_plan_destroy(p)


def test_noalloc_rejects_plans_beyond_the_static_scratch():
    """muon_step_noalloc checks the plan's workspace against its static scratch before any
    HIP call: the GPT-2-124M set (490 MiB) is refused with a message naming both sizes, the
    8-GPU share (61.2 MiB) fits, an empty plan is a no-op."""
    import seeded_inputs as si
    full = si.WORKLOADS["gpt2_124m"].shapes
    p = L.muon_plan_create([r for r, _ in full], [c for _, c in full], [0] * len(full),
                           [0] * len(full))
    try:
        assert L.muon_plan_workspace_size(p) > L.MUON_STATIC_SCRATCH_BYTES
        with pytest.raises(L.MuonError) as e:
            L.muon_step_noalloc(p, None, len(full), L.muon_config_default(), 0)
        assert e.value.status == L.MUON_ERR_WORKSPACE
        assert str(L.MUON_STATIC_SCRATCH_BYTES) in str(e.value)
    finally:
        L.muon_plan_destroy(p)
    share = si.WORKLOADS["gpt2_124m_share8"].shapes
    p = L.muon_plan_create([r for r, _ in share], [c for _, c in share], [0] * len(share),
                           [0] * len(share))
    try:
        assert 0 < L.muon_plan_workspace_size(p) <= L.MUON_STATIC_SCRATCH_BYTES
    finally:
        L.muon_plan_destroy(p)
    p = L.muon_plan_create([], [], [], [])
    L.muon_step_noalloc(p, None, 0, L.muon_config_default(), 0)
    L.muon_plan_destroy(p)
