"""The four-block work-item map of the symmetric products (ns_quad_bf16.hip), checked on the
host: tests/host_cpp/quad_items_check.cpp compiles the kernel source with hipcc and walks
every item of groups of 1-50 matrices, 256 to 2048 wide. Every upper 128x128 block must be
stored by exactly one wave, every index must be in range, and the slots a wave multiplies
must hold its block's row and column panels."""
import os
import subprocess

import pytest

from orthogonalized_momentum_optimizer_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_every_upper_block_is_computed_once(tmp_path):
    cc = build.hipcc()
    if not os.path.exists(cc):
        pytest.skip("hipcc is not available")
    exe = str(tmp_path / "quad_items_check")
    cmd = [cc, "--offload-arch=gfx950", "-std=c++17", "-O1",
           "-I", build.CSRC, "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "host_cpp", "quad_items_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-2000:]
    assert "quad items ok" in r.stdout
