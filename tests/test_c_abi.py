"""The C ABI from a plain C99 program (tests/c_abi/abi_check.c), compiled with gcc against
include/ and linked with libmuon.so. Only host-side validation paths run, so no GPU is
needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "orthogonalized_momentum_optimizer_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not available")
def test_c_program_uses_the_abi(tmp_path):
    lib = os.path.join(PKG, "libmuon.so")
    assert os.path.exists(lib), "build the library first"
    exe = str(tmp_path / "abi_check")
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c_abi", "abi_check.c"), "-o", exe,
           "-L", PKG, "-lmuon", "-Wl,-rpath," + PKG,
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi ok" in r.stdout
