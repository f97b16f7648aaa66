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


def test_traffic_record_tracks_its_source():
    # the committed apply record names the current source's hash and a positive byte count
    t = bench.measured_traffic("apply", "gpt2_124m")
    assert t is not None and t > 0
    # no record for a workload that has none
    assert bench.measured_traffic("apply", "attn_768") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "--gpus 1" in r.stderr
