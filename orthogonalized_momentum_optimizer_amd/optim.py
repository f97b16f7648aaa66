"""PyTorch-facing wrappers of the C ABI: a plan holder, the Newton-Schulz function, the
``Muon`` optimizer for the weight matrices and the ``CautiousAdam`` optimizer for the other
parameters.

The optimizer mirrors the constructor of page
"深入解析KellerJordan/modded-nanogpt中的训练架构与优化技术" (section
"Muon优化器：动量正交化技术", subsection "核心算法"): ``Muon(params, lr=0.02,
momentum=0.95, nesterov=True, ns_steps=5)``, with per-parameter "update buffers" (the
fp32 momentum). PyTorch supplies device memory and the current stream; the step itself
runs entirely in libmuon.so.
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence

import torch

from . import _lib as L

_DT = {torch.bfloat16: L.MUON_DT_BF16, torch.float32: L.MUON_DT_F32}
_PREC = {"bf16": L.MUON_NS_BF16, "f32": L.MUON_NS_F32_DEBUG}


def dtype_code(dt: torch.dtype) -> int:
    if dt not in _DT:
        raise TypeError(f"unsupported dtype {dt}: the library takes bfloat16 or float32")
    return _DT[dt]


def make_config(lr=0.02, beta=0.95, nesterov=True, ns_steps=5, abc=(3.4445, -4.7750, 2.0315),
                eps=1e-7, schedule=None, row_equalize=False, row_beta=0.95,
                row_eps=1e-8) -> L.muon_config:
    """A muon_config. ``schedule``: None, or ns_steps (a, b, c) triples, one per round.
    ``row_equalize``: apply the per-row energy equaliser (state buffers passed to the step)."""
    cfg = L.muon_config_default()
    cfg.lr, cfg.beta, cfg.nesterov, cfg.ns_steps = lr, beta, int(bool(nesterov)), int(ns_steps)
    cfg.a, cfg.b, cfg.c = abc
    cfg.eps = eps
    cfg.row_equalize, cfg.row_beta, cfg.row_eps = int(bool(row_equalize)), row_beta, row_eps
    if schedule is not None:
        flat = [float(x) for triple in schedule for x in triple]
        if len(flat) != 3 * int(ns_steps):
            raise ValueError("schedule must hold ns_steps (a, b, c) triples")
        arr = (ctypes.c_float * max(len(flat), 1))(*flat)
        cfg.schedule = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
        cfg._schedule_keepalive = arr   # the array lives as long as the config
    return cfg


def _stream_handle(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


class MuonPlan:
    """A plan of the library for a fixed list of matrix shapes and dtypes, with its device
    workspace (allocated once here, never inside a step)."""

    def __init__(self, shapes: Sequence[Sequence[int]], param_dtypes: Sequence[torch.dtype],
                 grad_dtypes: Sequence[torch.dtype], precision: str = "bf16",
                 device: Optional[torch.device] = None, workspace: bool = True,
                 streams: int = L.MUON_MAX_STREAMS, fused: bool = True):
        """``workspace=False``: no workspace is allocated; only ``step_noalloc`` (the
        library's static device scratch) can then run the step. ``streams``: shape groups a
        step may run concurrently (muon_plan_set_concurrency; 1 runs them in sequence).
        ``fused``: all rounds as one launch where the plan allows it (muon_plan_set_fused)."""
        self.shapes = [tuple(int(x) for x in s) for s in shapes]
        self.pdt = [dtype_code(d) for d in param_dtypes]
        self.gdt = [dtype_code(d) for d in grad_dtypes]
        self.precision = precision
        self.handle = L.muon_plan_create([s[0] for s in self.shapes], [s[1] for s in self.shapes],
                                         self.pdt, self.gdt, _PREC[precision])
        self.ws_bytes = L.muon_plan_workspace_size(self.handle)
        dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.workspace = None
        if workspace:
            # 256-byte alignment: torch's caching allocator returns 512-byte aligned blocks
            self.workspace = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=dev)
            assert self.workspace.data_ptr() % 256 == 0
        self._mats = None
        self._mats_key = None
        L.muon_plan_set_fused(self.handle, fused)
        with torch.cuda.device(dev):
            L.muon_plan_set_concurrency(self.handle, streams)

    def set_concurrency(self, streams: int):
        L.muon_plan_set_concurrency(self.handle, streams)

    def set_fused(self, enable: bool):
        L.muon_plan_set_fused(self.handle, enable)

    def close(self):
        if getattr(self, "handle", None):
            L.muon_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _matrices(self, params, grads, moms, outs, row_vars=None):
        n = len(self.shapes)
        outs = outs if outs is not None else [None] * n
        row_vars = row_vars if row_vars is not None else [None] * n
        key = tuple((p.data_ptr(), g.data_ptr(), m.data_ptr(), o.data_ptr() if o is not None else 0,
                     v.data_ptr() if v is not None else 0)
                    for p, g, m, o, v in zip(params, grads, moms, outs, row_vars))
        if key != self._mats_key:
            ents = []
            for i, (p, g, m, o, v) in enumerate(zip(params, grads, moms, outs, row_vars)):
                r, c = self.shapes[i]
                for t in (p, g, m) + ((o,) if o is not None else ()):
                    if tuple(t.shape) != (r, c) or not t.is_contiguous() or not t.is_cuda:
                        raise ValueError(f"matrix {i}: tensors must be contiguous CUDA "
                                         f"{r}x{c} (got {tuple(t.shape)})")
                if m.dtype != torch.float32 or (o is not None and o.dtype != torch.float32):
                    raise TypeError(f"matrix {i}: momentum and update_out must be float32")
                if v is not None and (v.numel() != r or v.dtype != torch.float32 or
                                      not v.is_contiguous() or not v.is_cuda):
                    raise ValueError(f"matrix {i}: row_var must be a contiguous CUDA float32 "
                                     f"tensor of {r} elements")
                ents.append((p.data_ptr(), g.data_ptr(), m.data_ptr(),
                             o.data_ptr() if o is not None else None, r, c,
                             dtype_code(p.dtype), dtype_code(g.dtype),
                             v.data_ptr() if v is not None else None))
            self._mats = L.make_matrices(ents)
            self._mats_key = key
        return self._mats

    def set_profiling(self, enable: bool):
        L.muon_plan_set_profiling(self.handle, enable)

    def read_profile(self) -> dict:
        return L.muon_plan_read_profile(self.handle)

    def step(self, params: Sequence[torch.Tensor], grads: Sequence[torch.Tensor],
             moms: Sequence[torch.Tensor], cfg: L.muon_config,
             outs: Optional[Sequence[Optional[torch.Tensor]]] = None,
             stream: Optional[torch.cuda.Stream] = None,
             row_vars: Optional[Sequence[torch.Tensor]] = None) -> None:
        """``row_vars``: per matrix a float32 tensor of ``rows`` elements (the row equaliser's
        state), needed when ``cfg.row_equalize`` is set."""
        n = len(self.shapes)
        if not (len(params) == len(grads) == len(moms) == n):
            raise ValueError(f"expected {n} params, grads and momentum buffers")
        if row_vars is not None and len(row_vars) != n:
            raise ValueError(f"expected {n} row_var buffers")
        mats = self._matrices(params, grads, moms, outs, row_vars) if n else None
        if self.workspace is None:
            raise RuntimeError("this plan has no workspace: use step_noalloc")
        L.muon_step(self.handle, mats, n, cfg, self.workspace.data_ptr(), self.ws_bytes,
                    _stream_handle(stream))

    def step_noalloc(self, params: Sequence[torch.Tensor], grads: Sequence[torch.Tensor],
                     moms: Sequence[torch.Tensor], cfg: L.muon_config,
                     outs: Optional[Sequence[Optional[torch.Tensor]]] = None,
                     stream: Optional[torch.cuda.Stream] = None,
                     row_vars: Optional[Sequence[torch.Tensor]] = None) -> None:
        """``step`` through muon_step_noalloc: the kernels' scratch is the library's static
        device array (at most MUON_STATIC_SCRATCH_BYTES of workspace), nothing is allocated."""
        n = len(self.shapes)
        if not (len(params) == len(grads) == len(moms) == n):
            raise ValueError(f"expected {n} params, grads and momentum buffers")
        if row_vars is not None and len(row_vars) != n:
            raise ValueError(f"expected {n} row_var buffers")
        mats = self._matrices(params, grads, moms, outs, row_vars) if n else None
        L.muon_step_noalloc(self.handle, mats, n, cfg, _stream_handle(stream))

    def newton_schulz(self, inputs: Sequence[torch.Tensor], outputs: Sequence[torch.Tensor],
                      cfg: L.muon_config, stream: Optional[torch.cuda.Stream] = None) -> None:
        n = len(self.shapes)
        if not (len(inputs) == len(outputs) == n):
            raise ValueError(f"expected {n} inputs and outputs")
        for i, (x, y) in enumerate(zip(inputs, outputs)):
            if (tuple(x.shape) != self.shapes[i] or tuple(y.shape) != self.shapes[i]
                    or not x.is_contiguous() or not y.is_contiguous()):
                raise ValueError(f"matrix {i}: contiguous {self.shapes[i]} tensors expected")
            if dtype_code(x.dtype) != self.gdt[i] or dtype_code(y.dtype) != self.pdt[i]:
                raise TypeError(f"matrix {i}: dtypes differ from the plan's")
        if self.workspace is None:
            raise RuntimeError("this plan has no workspace")
        L.muon_newton_schulz(self.handle, [x.data_ptr() for x in inputs],
                             [y.data_ptr() for y in outputs], cfg, self.workspace.data_ptr(),
                             self.ws_bytes, _stream_handle(stream))


def zeropower_via_newtonschulz5(G: torch.Tensor, steps: int = 5, precision: str = "bf16",
                                out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """NS(G / (||G||_F + eps)) for one 2-D CUDA tensor, through libmuon.so. The result has
    G's shape and ``out_dtype`` (bfloat16 like the pages' function)."""
    if G.dim() != 2:
        raise ValueError("G must be 2-D")
    G = G.contiguous()
    out = torch.empty(G.shape, dtype=out_dtype, device=G.device)
    plan = MuonPlan([G.shape], [out_dtype], [G.dtype], precision, G.device)
    plan.newton_schulz([G], [out], make_config(ns_steps=steps))
    # keep the workspace alive until the stream has passed the call
    torch.cuda.current_stream().synchronize()
    plan.close()
    return out


class Muon(torch.optim.Optimizer):
    """Muon: SGD-Nesterov momentum orthogonalised by Newton-Schulz, for 2-D (or stacked
    >= 3-D) weight matrices. Each >= 3-D parameter is treated as a stack of matrices over
    its last two dimensions. 1-D parameters are rejected (they belong to another optimizer).
    ``row_equalize`` adds the per-row energy equaliser of the NorMuon family between the
    orthogonalisation and the update (state: one float per row of every matrix).
    """

    def __init__(self, params, lr: float = 0.02, momentum: float = 0.95, nesterov: bool = True,
                 ns_steps: int = 5, precision: str = "bf16", row_equalize: bool = False,
                 row_beta: float = 0.95, row_eps: float = 1e-8):
        defaults = dict(lr=lr, momentum=momentum, nesterov=nesterov, ns_steps=ns_steps,
                        row_equalize=row_equalize, row_beta=row_beta, row_eps=row_eps)
        super().__init__(params, defaults)
        if precision not in _PREC:
            raise ValueError(f"precision must be one of {sorted(_PREC)}")
        self.precision = precision
        for group in self.param_groups:
            for p in group["params"]:
                if p.dim() < 2:
                    raise ValueError("Muon takes matrices only (2-D or stacked >= 3-D params)")
        self._plans = {}

    @staticmethod
    def _split(t: torch.Tensor) -> List[torch.Tensor]:
        if t.dim() == 2:
            return [t]
        flat = t.reshape(-1, t.shape[-2], t.shape[-1])
        return [flat[i] for i in range(flat.shape[0])]

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        for gi, group in enumerate(self.param_groups):
            params, grads, moms, rvars = [], [], [], []
            for p in group["params"]:
                if p.grad is None:
                    continue
                if not p.is_contiguous() or not p.grad.is_contiguous():
                    raise ValueError("Muon needs contiguous parameters and gradients")
                st = self.state[p]
                if "momentum_buffer" not in st:
                    st["momentum_buffer"] = torch.zeros(p.shape, dtype=torch.float32,
                                                        device=p.device)
                params += self._split(p)
                grads += self._split(p.grad)
                moms += self._split(st["momentum_buffer"])
                if group["row_equalize"]:
                    if "row_var" not in st:
                        st["row_var"] = torch.zeros(p.shape[:-1], dtype=torch.float32,
                                                    device=p.device)
                    rv = st["row_var"]
                    rvars += [rv] if rv.dim() == 1 else list(rv.reshape(-1, rv.shape[-1]))
            if not params:
                continue
            key = (gi, tuple((tuple(x.shape), x.dtype, g.dtype) for x, g in zip(params, grads)))
            plan = self._plans.get(key)
            if plan is None:
                plan = MuonPlan([x.shape for x in params], [x.dtype for x in params],
                                [g.dtype for g in grads], self.precision, params[0].device)
                self._plans[key] = plan
            cfg = make_config(lr=group["lr"], beta=group["momentum"],
                              nesterov=group["nesterov"], ns_steps=group["ns_steps"],
                              row_equalize=group["row_equalize"], row_beta=group["row_beta"],
                              row_eps=group["row_eps"])
            plan.step(params, grads, moms, cfg, row_vars=rvars if group["row_equalize"] else None)
        return loss


def make_adam_config(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0,
                     step=1) -> L.muon_adam_config:
    """A muon_adam_config; ``step`` is the index t >= 1 of the step in the bias corrections."""
    cfg = L.muon_adam_config_default()
    cfg.lr, cfg.beta1, cfg.beta2 = lr, betas[0], betas[1]
    cfg.eps, cfg.weight_decay, cfg.step = eps, weight_decay, int(step)
    return cfg


def cautious_adam_step(params: Sequence[torch.Tensor], grads: Sequence[torch.Tensor],
                       exp_avgs: Sequence[torch.Tensor], exp_avg_sqs: Sequence[torch.Tensor],
                       cfg: L.muon_adam_config, wd_muls: Optional[Sequence[float]] = None,
                       stream: Optional[torch.cuda.Stream] = None) -> None:
    """One cautious-Adam step of libmuon.so over contiguous CUDA tensors of any shape (p and g
    bfloat16 or float32, the two moments float32 and zero before step 1)."""
    n = len(params)
    if not (len(grads) == len(exp_avgs) == len(exp_avg_sqs) == n):
        raise ValueError("params, grads, exp_avgs and exp_avg_sqs must have the same length")
    wd_muls = [1.0] * n if wd_muls is None else list(wd_muls)
    if len(wd_muls) != n:
        raise ValueError("one wd_mul per tensor")
    ents = []
    for i, (p, g, m, v) in enumerate(zip(params, grads, exp_avgs, exp_avg_sqs)):
        for t in (p, g, m, v):
            if t.numel() != p.numel() or not t.is_contiguous() or not t.is_cuda:
                raise ValueError(f"tensor {i}: contiguous CUDA tensors of {p.numel()} "
                                 "elements expected")
        if m.dtype != torch.float32 or v.dtype != torch.float32:
            raise TypeError(f"tensor {i}: exp_avg and exp_avg_sq must be float32")
        ents.append((p.data_ptr(), g.data_ptr(), m.data_ptr(), v.data_ptr(), p.numel(),
                     dtype_code(p.dtype), dtype_code(g.dtype), float(wd_muls[i])))
    arr = L.make_adam_tensors(ents) if n else None
    L.muon_cautious_adam_step(arr, n, cfg, _stream_handle(stream))


class CautiousAdam(torch.optim.Optimizer):
    """Adam with cautious (sign-masked, decoupled) weight decay for the non-matrix
    parameters (embeddings, LM head, scalars), as in the record analysed at lqnn.cn,
    section 3.3. Each parameter group may carry ``wd_mul``, the multiplier of the base
    ``weight_decay`` for its tensors (the page's table uses 150 for embed / lm_head and 0 for
    scalars). The whole step runs in libmuon.so, one fused pass per dtype pair."""

    def __init__(self, params, lr: float = 1e-3, betas=(0.9, 0.999), eps: float = 1e-8,
                 weight_decay: float = 0.0, wd_mul: float = 1.0):
        defaults = dict(lr=lr, betas=tuple(betas), eps=eps, weight_decay=weight_decay,
                        wd_mul=wd_mul)
        super().__init__(params, defaults)

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        for group in self.param_groups:
            by_step = {}
            for p in group["params"]:
                if p.grad is None:
                    continue
                if not p.is_contiguous() or not p.grad.is_contiguous():
                    raise ValueError("CautiousAdam needs contiguous parameters and gradients")
                st = self.state[p]
                if "step" not in st:
                    st["step"] = 0
                    st["exp_avg"] = torch.zeros(p.shape, dtype=torch.float32, device=p.device)
                    st["exp_avg_sq"] = torch.zeros(p.shape, dtype=torch.float32,
                                                   device=p.device)
                st["step"] += 1
                by_step.setdefault(st["step"], []).append(p)
            for t, ps in by_step.items():
                cfg = make_adam_config(group["lr"], group["betas"], group["eps"],
                                       group["weight_decay"], t)
                cautious_adam_step(ps, [p.grad for p in ps],
                                   [self.state[p]["exp_avg"] for p in ps],
                                   [self.state[p]["exp_avg_sq"] for p in ps], cfg,
                                   [group["wd_mul"]] * len(ps))
        return loss
