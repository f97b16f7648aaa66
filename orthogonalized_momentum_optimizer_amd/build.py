"""Builds libmuon.so (the HIP kernels and the C ABI of include/*.h) for gfx950 in place.

    python -m orthogonalized_momentum_optimizer_amd.build

Every source under csrc/ is compiled with hipcc for gfx950 only and linked into
orthogonalized_momentum_optimizer_amd/libmuon.so, except mfma_loop.hip, a measurement kernel
for bench.py that goes into libmuon_mfma_loop.so. Objects go to _build/ at the repository
root. The library links against the HIP runtime by its soname, so inside a process that has
already loaded PyTorch's HIP runtime the library binds to that same runtime.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmuon.so")
# measurement only, a library of its own (bench.py's matrix-core issue bound)
PROBE_LIB = os.path.join(PKG, "libmuon_mfma_loop.so")
PROBE_SOURCES = ["mfma_loop.hip"]

SOURCES = ["plan.hip", "elementwise.hip", "ns_gemm_bf16.hip", "ns_sym256_bf16.hip",
           "ns_quad_bf16.hip", "ns_apply_bf16.hip", "ns_fused_bf16.hip", "ns_gemm_f32.hip",
           "cautious_adam.hip", "noalloc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # keep hipcc from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libmuon.so")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in (r.stderr or "").splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []

    def one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        msg = _run([cc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES) + len(PROBE_SOURCES))) as ex:
        objs = list(ex.map(one, SOURCES + PROBE_SOURCES))
    for lib, part in ((LIB, objs[:len(SOURCES)]), (PROBE_LIB, objs[len(SOURCES):])):
        tmp = lib + ".tmp"
        _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp,
              *part])
        os.replace(tmp, lib)
        if verbose:
            print(f"built {lib}")
    return LIB


def device_asm(src: str) -> str:
    """Compiles one source under csrc/ to gfx950 assembly (device code only, the library's
    flags) into _build/asm/ and returns the path; reused while the source files are unchanged."""
    import hashlib
    out_dir = os.path.join(BUILD, "asm")
    os.makedirs(out_dir, exist_ok=True)
    h = hashlib.sha256()
    headers = [os.path.join(INCLUDE, h) for h in sorted(os.listdir(INCLUDE))]
    for name in sorted(os.listdir(CSRC)) + headers:
        path = name if os.path.isabs(name) else os.path.join(CSRC, name)
        with open(path, "rb") as f:
            h.update(f.read())
    out = os.path.join(out_dir, f"{os.path.splitext(src)[0]}-{h.hexdigest()[:16]}.s")
    if not os.path.exists(out):
        tmp = out + ".tmp"
        _run([hipcc(), *HIPCC_FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, src),
              "-o", tmp])
        os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose=True)
