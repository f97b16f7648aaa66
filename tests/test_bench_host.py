"""bench.py's host-side arithmetic and checks (no GPU): the algorithmic work it divides by,
the traffic record it reads from profiles/, and its refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

import seeded_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_kind_work_matches_the_nominal_count():
    wl = si.WORKLOADS["gpt2_124m"]
    w = bench.kind_work(wl)
    # gram + poly + apply = 5 x sum(4 m^2 n + 2 m^3), the metric's nominal count
    assert abs((w["gram"] + w["poly"] + w["apply"]) - wl.ns_flops_per_step()) < 1.0
    # per round, apply = gram = 2 m^2 n and poly = 2 m^3 (m = 768 for every matrix)
    assert w["apply"] == w["gram"]
    assert w["poly"] == 5 * 72 * 2.0 * 768 ** 3
    # bf16 W and G with fp32 momentum: momentum 2 + 8 bytes, update 2 + 2 bytes per element
    assert w["momentum"] == 10.0 * wl.elements()
    assert w["update"] == 4.0 * wl.elements()


def test_adam_bytes_per_element():
    assert bench.adam_bytes_per_element("bf16", "bf16") == 22   # 2+2+4+4 read, 2+4+4 written
    assert bench.adam_bytes_per_element("f32", "f32") == 28   # 4+4+4+4 read, 4+4+4 written
    assert bench.adam_bytes_per_element("f32", "bf16") == 26   # 4+2+4+4 read, 4+4+4 written


def test_traffic_record_tracks_its_source(tmp_path, monkeypatch):
    """A traffic record counts only while the source it names by hash is unchanged."""
    import hashlib
    csrc = tmp_path / "orthogonalized_momentum_optimizer_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    src = csrc / "ns_apply_bf16.hip"
    src.write_text("// kernel source\n")
    digest = hashlib.sha256(src.read_bytes()).hexdigest()
    (tmp_path / "profiles" / "apply_gpt2_124m_traffic.md").write_text(
        f"traffic_bytes_per_launch: 1.5e8\nsource_sha256: {digest}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("apply", "gpt2_124m") == 1.5e8
    assert bench.measured_traffic("apply", "attn_768") is None     # no record
    src.write_text("// kernel source, changed\n")
    assert bench.measured_traffic("apply", "gpt2_124m") is None    # stale record


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "--gpus 1" in r.stderr


def test_cpu_baseline_times_the_oracle_only(monkeypatch):
    """Input generation stays outside the timed region: with drawing made slow on purpose
    (0.3 s per tensor) the reported rate still reflects the oracle's own time."""
    import time as _time
    wl = si.custom([(64, 256), (256, 64)], dtype="f32", steps=1, cfg_id=140, grad_std=1.0)
    real_w, real_g = si.weight, si.grad

    def slow_weight(*a):
        _time.sleep(0.3)
        return real_w(*a)

    def slow_grad(*a):
        _time.sleep(0.3)
        return real_g(*a)

    monkeypatch.setattr(bench.si, "weight", slow_weight)
    monkeypatch.setattr(bench.si, "grad", slow_grad)
    out = bench.cpu_baseline(wl, budget_s=5.0)
    # two tiny matrices: a whole step takes milliseconds in the oracle; timing the 1.2 s of
    # drawing per step would report below 0.84 steps/s (the bound leaves room for a loaded
    # host)
    assert out["value"] > 2.0, out
    assert "not timed" in out["sample"]
    assert out["kind"] == "oracle" and out["cores"] >= 1


def test_product_launch_model_matches_the_launches_of_the_gpt2_124m_set():
    """The grids the matrix-core bound replays are those the library launches for the
    GPT-2-124M set on 256 compute units (the kernel trace shows 1008- and 504-block products
    of 128x128 tiles and 216 persistent apply blocks)."""
    got = bench.product_launches(si.WORKLOADS["gpt2_124m"], 256, fused=False)
    assert got == [
        ("gram", (48, 768, 768), 1008, 4, 24, 65536),
        ("poly", (48, 768, 768), 1008, 4, 24, 65536),
        ("apply", (48, 768, 768), 216, 16, 48, 131072),
        ("gram", (24, 768, 3072), 504, 4, 96, 65536),
        ("poly", (24, 768, 3072), 504, 4, 24, 65536),
        ("apply", (24, 768, 3072), 216, 16, 96, 131072),
    ]
    # the apply grids issue exactly the nominal 2 m^2 n flops of their group (every block
    # takes the same number of 256x256 tiles); the symmetric products one block per upper
    # 128x128 tile
    mfma_flops = 2 * 32 * 32 * 16
    for kind, (b, mp, np_), blocks, nacc, iters, _ in got:
        if kind == "apply":
            assert blocks * 4 * iters * 2 * nacc * mfma_flops == 2 * b * mp * mp * np_
        else:
            assert blocks == b * (mp // 128) * (mp // 128 + 1) // 2
    assert bench.product_launches(si.WORKLOADS["gpt2_124m_share8"], 256) is None
    # all rounds in one launch: 252 + 126 four-block items of K = 768 / 3072 (Gram) and
    # 768 (polynomial), 432 + 864 apply tiles of K = 768, five rounds over 256 blocks
    units = 252 * (24 + 24) + 432 * 24 + 126 * (96 + 24) + 864 * 24
    assert bench.product_launches(si.WORKLOADS["gpt2_124m"], 256) == [
        ("rounds", "all", 256, 16, -(-5 * units // 256), 131072)]
    # sets with more than 8 apply tiles per compute unit per round keep one launch per
    # product: the tall stress set (96 x 768x3072 wide, 13.5 tiles per unit)
    assert bench.fused_rounds(bench.shape_groups(si.WORKLOADS["tall_stress"]), 5) is False
    assert bench.fused_rounds(bench.shape_groups(si.WORKLOADS["gpt2_124m"]), 5) is True
    assert bench.fused_rounds(bench.shape_groups(si.WORKLOADS["gpt2_124m"]), 5, cus=304) is False
