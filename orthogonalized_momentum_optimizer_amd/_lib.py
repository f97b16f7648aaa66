"""ctypes binding of libmuon.so (the C ABI of include/muon.h and include/cautious_adam.h),
with the same names.

Only argument marshalling happens here: every step of the optimizer runs in the HIP
kernels of the library. PyTorch's HIP runtime is loaded first (``import torch``) so the
library binds to that same runtime and can use torch's device pointers and streams.
A missing or unloadable library is an error, never a fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import torch  # noqa: F401  (loads the HIP runtime the library must share)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmuon.so")

MUON_OK = 0
MUON_ERR_INVALID_ARG = -1
MUON_ERR_UNSUPPORTED = -2
MUON_ERR_WORKSPACE = -3
MUON_ERR_HIP = -4

MUON_DT_BF16 = 0
MUON_DT_F32 = 1
MUON_NS_BF16 = 0
MUON_NS_F32_DEBUG = 1

KERNEL_KINDS = ("momentum", "norm", "gram", "poly", "apply", "update", "roweq", "rounds")

EXPORTED = (
    "muon_config_default", "muon_plan_create", "muon_plan_workspace_size", "muon_step",
    "muon_newton_schulz", "muon_plan_destroy", "muon_plan_set_profiling",
    "muon_plan_read_profile", "muon_status_string", "muon_last_error",
    "muon_adam_config_default", "muon_cautious_adam_step", "muon_step_noalloc",
    "muon_plan_set_concurrency", "muon_plan_set_fused",
)
MUON_MAX_STREAMS = 4
MUON_STATIC_SCRATCH_BYTES = 64 << 20


class MuonError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


class muon_matrix(ctypes.Structure):
    _fields_ = [
        ("param", ctypes.c_void_p),
        ("grad", ctypes.c_void_p),
        ("momentum", ctypes.c_void_p),
        ("update_out", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("param_dtype", ctypes.c_int),
        ("grad_dtype", ctypes.c_int),
        ("row_var", ctypes.c_void_p),
    ]


class muon_config(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float),
        ("beta", ctypes.c_float),
        ("nesterov", ctypes.c_int),
        ("ns_steps", ctypes.c_int),
        ("a", ctypes.c_float),
        ("b", ctypes.c_float),
        ("c", ctypes.c_float),
        ("eps", ctypes.c_float),
        ("schedule", ctypes.POINTER(ctypes.c_float)),
        ("row_equalize", ctypes.c_int),
        ("row_beta", ctypes.c_float),
        ("row_eps", ctypes.c_float),
    ]


class muon_adam_tensor(ctypes.Structure):
    _fields_ = [
        ("param", ctypes.c_void_p),
        ("grad", ctypes.c_void_p),
        ("exp_avg", ctypes.c_void_p),
        ("exp_avg_sq", ctypes.c_void_p),
        ("numel", ctypes.c_int64),
        ("param_dtype", ctypes.c_int),
        ("grad_dtype", ctypes.c_int),
        ("wd_mul", ctypes.c_float),
    ]


class muon_adam_config(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float),
        ("beta1", ctypes.c_float),
        ("beta2", ctypes.c_float),
        ("eps", ctypes.c_float),
        ("weight_decay", ctypes.c_float),
        ("step", ctypes.c_int64),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if libmuon.so has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m orthogonalized_momentum_optimizer_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    L.muon_config_default.argtypes = [ctypes.POINTER(muon_config)]
    L.muon_config_default.restype = None
    L.muon_plan_create.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(i64), ctypes.POINTER(i64),
                                   ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                   i64, ctypes.c_int]
    L.muon_plan_create.restype = ctypes.c_int
    L.muon_plan_workspace_size.argtypes = [vp]
    L.muon_plan_workspace_size.restype = sz
    L.muon_step.argtypes = [vp, ctypes.POINTER(muon_matrix), i64, ctypes.POINTER(muon_config),
                            vp, sz, vp]
    L.muon_step.restype = ctypes.c_int
    L.muon_step_noalloc.argtypes = [vp, ctypes.POINTER(muon_matrix), i64,
                                    ctypes.POINTER(muon_config), ctypes.c_void_p]
    L.muon_step_noalloc.restype = ctypes.c_int
    L.muon_newton_schulz.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), i64,
                                     ctypes.POINTER(muon_config), vp, sz, vp]
    L.muon_newton_schulz.restype = ctypes.c_int
    L.muon_plan_destroy.argtypes = [vp]
    L.muon_plan_destroy.restype = None
    L.muon_plan_set_profiling.argtypes = [vp, ctypes.c_int]
    L.muon_plan_set_profiling.restype = ctypes.c_int
    L.muon_plan_set_concurrency.argtypes = [vp, ctypes.c_int]
    L.muon_plan_set_concurrency.restype = ctypes.c_int
    L.muon_plan_set_fused.argtypes = [vp, ctypes.c_int]
    L.muon_plan_set_fused.restype = ctypes.c_int
    L.muon_plan_read_profile.argtypes = [vp, ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(i64), ctypes.c_int]
    L.muon_plan_read_profile.restype = ctypes.c_int
    L.muon_adam_config_default.argtypes = [ctypes.POINTER(muon_adam_config)]
    L.muon_adam_config_default.restype = None
    L.muon_cautious_adam_step.argtypes = [ctypes.POINTER(muon_adam_tensor), i64,
                                          ctypes.POINTER(muon_adam_config), vp]
    L.muon_cautious_adam_step.restype = ctypes.c_int
    L.muon_status_string.argtypes = [ctypes.c_int]
    L.muon_status_string.restype = ctypes.c_char_p
    L.muon_last_error.argtypes = []
    L.muon_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().muon_status_string(int(status)).decode()


def muon_last_error() -> str:
    return lib().muon_last_error().decode()


def _check(status: int) -> None:
    if status != MUON_OK:
        raise MuonError(status, muon_last_error())


def muon_status_string(status: int) -> str:
    return status_string(status)


def muon_config_default() -> muon_config:
    cfg = muon_config()
    lib().muon_config_default(ctypes.byref(cfg))
    return cfg


def muon_plan_create(rows: Sequence[int], cols: Sequence[int], param_dtype: Sequence[int],
                     grad_dtype: Sequence[int], precision: int = MUON_NS_BF16) -> int:
    n = len(rows)
    if not (len(cols) == len(param_dtype) == len(grad_dtype) == n):
        raise ValueError("rows, cols, param_dtype and grad_dtype must have the same length")
    plan = ctypes.c_void_p()
    arr = lambda t, xs: (t * max(n, 1))(*xs)  # noqa: E731
    _check(lib().muon_plan_create(ctypes.byref(plan), arr(ctypes.c_int64, rows),
                                  arr(ctypes.c_int64, cols), arr(ctypes.c_int, param_dtype),
                                  arr(ctypes.c_int, grad_dtype), n, int(precision)))
    return plan.value


def muon_plan_workspace_size(plan: int) -> int:
    return int(lib().muon_plan_workspace_size(plan))


def muon_plan_destroy(plan: int) -> None:
    lib().muon_plan_destroy(plan)


def muon_step(plan: int, mats, n: int, cfg: muon_config, workspace: int, workspace_bytes: int,
              stream: int) -> None:
    """``mats``: a ctypes array of muon_matrix (or None when n == 0)."""
    _check(lib().muon_step(plan, mats, n, ctypes.byref(cfg), workspace, workspace_bytes, stream))


def muon_step_noalloc(plan: int, mats, n: int, cfg: muon_config, stream: int) -> None:
    """muon_step with the library's static device scratch instead of a workspace."""
    _check(lib().muon_step_noalloc(plan, mats, n, ctypes.byref(cfg), stream))


def muon_newton_schulz(plan: int, inputs: Sequence[int], outputs: Sequence[int],
                       cfg: muon_config, workspace: int, workspace_bytes: int,
                       stream: int) -> None:
    n = len(inputs)
    ins = (ctypes.c_void_p * max(n, 1))(*inputs)
    outs = (ctypes.c_void_p * max(n, 1))(*outputs)
    _check(lib().muon_newton_schulz(plan, ins, outs, n, ctypes.byref(cfg), workspace,
                                    workspace_bytes, stream))


def muon_plan_set_profiling(plan: int, enable: bool) -> None:
    _check(lib().muon_plan_set_profiling(plan, 1 if enable else 0))


def muon_plan_set_concurrency(plan: int, streams: int) -> None:
    _check(lib().muon_plan_set_concurrency(plan, int(streams)))


def muon_plan_set_fused(plan: int, enable: bool) -> None:
    _check(lib().muon_plan_set_fused(plan, 1 if enable else 0))


def muon_plan_read_profile(plan: int) -> dict:
    k = len(KERNEL_KINDS)
    ms = (ctypes.c_double * k)()
    n = (ctypes.c_int64 * k)()
    _check(lib().muon_plan_read_profile(plan, ms, n, k))
    return {name: (ms[i], n[i]) for i, name in enumerate(KERNEL_KINDS)}


def make_matrices(entries) -> ctypes.Array:
    """entries: iterable of (param_ptr, grad_ptr, momentum_ptr, out_ptr, rows, cols, pdt, gdt
    [, row_var_ptr])."""
    entries = list(entries)
    arr = (muon_matrix * max(len(entries), 1))()
    for i, e in enumerate(entries):
        arr[i] = muon_matrix(*e)
    return arr


def muon_adam_config_default() -> muon_adam_config:
    cfg = muon_adam_config()
    lib().muon_adam_config_default(ctypes.byref(cfg))
    return cfg


def muon_cautious_adam_step(tensors, n: int, cfg: muon_adam_config, stream: int) -> None:
    """``tensors``: a ctypes array of muon_adam_tensor (or None when n == 0)."""
    _check(lib().muon_cautious_adam_step(tensors, n, ctypes.byref(cfg), stream))


def make_adam_tensors(entries) -> ctypes.Array:
    """entries: iterable of (param, grad, exp_avg, exp_avg_sq, numel, pdt, gdt, wd_mul)."""
    entries = list(entries)
    arr = (muon_adam_tensor * max(len(entries), 1))()
    for i, e in enumerate(entries):
        arr[i] = muon_adam_tensor(*e)
    return arr
