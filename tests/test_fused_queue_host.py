"""The single launch's work queues (ns_fused_bf16.hip), checked on the host:
tests/host_cpp/fused_queue_check.cpp compiles the kernel source with hipcc and walks every
XCD's queue in claim order through the kernel's own decode and item_deps, for the GPT-2-124M
groups and 150 seeded sets of 1-4 groups (8-40 matrices, 256-1536 rows, up to 1792 more
columns, 1-16 rounds). Every product must be made exactly once, every item must wait for the
counters of the matrices it reads with the count those counters receive, and every item that
signals a counter must come earlier in the same queue: the launch's progress argument.

The checker's own power is shown on copies of the source with one planted mistake each
(compiled for the host only): a Gram item waiting on its own round's apply counters, a
polynomial item waiting on one of its two matrices, an apply tile waiting on the Gram counter,
a wrong count, and the rounds taken in reverse queue order. Each must fail."""
import os
import shutil
import subprocess

import pytest

from orthogonalized_momentum_optimizer_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(build.CSRC, "ns_fused_bf16.hip")

MUTANTS = {
    "gram_waits_on_own_round": (
        "((size_t)PH_APPLY * F.rounds + it.r - 1) * row;",
        "((size_t)PH_APPLY * F.rounds + it.r) * row;"),
    "poly_waits_on_one_matrix": ("d.c[1] = c + m2;", "d.c[1] = c + m0;"),
    "apply_waits_on_gram": (
        "d.c[0] = G.cnt + ((size_t)PH_POLY * F.rounds + it.r) * row + (x + 8 * j);",
        "d.c[0] = G.cnt + ((size_t)PH_GRAM * F.rounds + it.r) * row + (x + 8 * j);"),
    "apply_count_per_tile": ("4u * G.tiles_m * G.tiles_n;", "2u * G.tiles_m * G.tiles_n;"),
    "rounds_reversed": (
        "  it.r = idx / per_round;\n  int rem = idx - it.r * per_round;",
        "  const int rr = idx / per_round;\n  int rem = idx - rr * per_round;\n"
        "  it.r = F.rounds - 1 - rr;"),
}


def _hipcc():
    cc = build.hipcc()
    if not os.path.exists(cc):
        pytest.skip("hipcc is not available")
    return cc


def _build_and_run(cc, csrc, exe):
    cmd = [cc, "--offload-arch=gfx950", "-std=c++17", "-O1", "-I", csrc,
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "host_cpp", "fused_queue_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, HIP_VISIBLE_DEVICES="")
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)


def test_queues_keep_the_progress_order(tmp_path):
    r = _build_and_run(_hipcc(), build.CSRC, str(tmp_path / "fused_queue_check"))
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-2000:]
    assert "fused queues ok" in r.stdout


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_queue_mistake_is_caught(tmp_path, name):
    cc = _hipcc()
    csrc = tmp_path / "csrc"
    shutil.copytree(build.CSRC, csrc)
    old, new = MUTANTS[name]
    path = csrc / "ns_fused_bf16.hip"
    text = path.read_text()
    assert text.count(old) == 1, f"{name}: the planted line no longer matches the source"
    path.write_text(text.replace(old, new))
    r = _build_and_run(cc, str(csrc), str(tmp_path / "fused_queue_check"))
    assert r.returncode != 0 and "fused queues ok" not in r.stdout, (name, r.stdout[-2000:])
