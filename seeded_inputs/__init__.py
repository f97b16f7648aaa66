"""Seeded synthetic inputs for the Muon step: the five workloads and their tensors.

This module is shared by the tests, the benchmark and the CPU oracle's callers. It holds
no part of the optimizer's arithmetic: it only describes the matrix sets and draws their
initial weights and per-step gradients from seeded generators.

Every draw comes from ``numpy.random.Generator(PCG64(SeedSequence([cfg_id, kind, index,
step])))`` with kind 0 = weights, 1 = gradients. Values are drawn in float64, rounded to
float32 by numpy and, for bf16 tensors, rounded once more to bfloat16 by torch (round to
nearest even). The stored values are what both the GPU path and the oracle receive.

Workloads (the matrix shapes of GPT-2-style models; the pages train GPT-2 124M and
1.5B, and their hidden matrices are the ones the Muon optimizer updates):

  gpt2_tiny_fp32   1 x 64x256, fp32 W and G; G ~ N(0, 1) drawn once and reused every step
  attn_768         1 x 768x768 bf16; G ~ N(0, 1e-3) fresh per step
  gpt2_124m        12 layers x (Q, K, V, O 768x768; fc 3072x768; proj 768x3072) bf16
  tall_stress      48 x 3072x768 + 48 x 768x3072 bf16; heavy-tailed gradient rows
  gpt2_1p5b        48 layers x (4 x 1600x1600; fc 6400x1600; proj 1600x6400) bf16
  gpt2_124m_shareN the matrices of gpt2_124m that rank 0 of N GPUs owns (N = 2, 4, 8) when
                   whole matrices are dealt out round-robin within each size group (one GPU's
                   share of a data-parallel step, at its real shapes); fresh draws

W ~ N(0, 0.02) everywhere (0.02 is the standard deviation). The heavy-tailed rows of
``tall_stress`` are g_ij = 1e-3 * |t_i| * z_ij with t_i ~ Student-t(3) per row and
z_ij ~ N(0, 1).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

KIND_WEIGHT = 0
KIND_GRAD = 1


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    shapes: Tuple[Tuple[int, int], ...]      # (rows, cols) per matrix, original orientation
    dtype: str                                # "bf16" or "f32" for W and G
    steps: int
    grad_std: float
    reuse_grad: bool = False                  # one gradient drawn once and reused every step
    heavy_tailed_rows: bool = False
    iid_t3_entries: bool = False              # every entry grad_std * Student-t(3), independent
    labels: Tuple[str, ...] = field(default=())

    @property
    def n(self) -> int:
        return len(self.shapes)

    def elements(self) -> int:
        return int(sum(r * c for r, c in self.shapes))

    def ns_flops_per_step(self, ns_steps: int = 5) -> float:
        """Nominal Newton-Schulz flops of one step: ns_steps * sum(4 m^2 n + 2 m^3), m <= n."""
        tot = 0.0
        for r, c in self.shapes:
            m, n = min(r, c), max(r, c)
            tot += 4.0 * m * m * n + 2.0 * m ** 3
        return ns_steps * tot


def _gpt2_layer_shapes(d: int):
    four = [(d, d)] * 4
    return four + [(4 * d, d), (d, 4 * d)], ["q", "k", "v", "o", "fc", "proj"]


def _build() -> dict:
    w = {}
    w["gpt2_tiny_fp32"] = Workload("gpt2_tiny_fp32", 0, ((64, 256),), "f32", 3, 1.0,
                                   reuse_grad=True, labels=("m0",))
    w["attn_768"] = Workload("attn_768", 1, ((768, 768),), "bf16", 10, 1e-3, labels=("o",))
    s, lab = _gpt2_layer_shapes(768)
    w["gpt2_124m"] = Workload("gpt2_124m", 2, tuple(s * 12), "bf16", 20, 1e-3,
                              labels=tuple(f"l{i}.{x}" for i in range(12) for x in lab))
    tall = [(3072, 768)] * 48 + [(768, 3072)] * 48
    w["tall_stress"] = Workload("tall_stress", 3, tuple(tall), "bf16", 20, 1e-3,
                                heavy_tailed_rows=True,
                                labels=tuple([f"fc{i}" for i in range(48)] +
                                             [f"proj{i}" for i in range(48)]))
    s, lab = _gpt2_layer_shapes(1600)
    w["gpt2_1p5b"] = Workload("gpt2_1p5b", 4, tuple(s * 48), "bf16", 10, 1e-3,
                              labels=tuple(f"l{i}.{x}" for i in range(48) for x in lab))
    full = w["gpt2_124m"]
    for cid, world in ((5, 2), (6, 4), (7, 8)):
        own = owned_indices(full.shapes, world, 0)
        name = f"gpt2_124m_share{world}"
        w[name] = Workload(name, cid, tuple(full.shapes[i] for i in own), "bf16", 20, 1e-3,
                           labels=tuple(full.labels[i] for i in own))
    return w


def owned_indices(shapes, world: int, rank: int) -> List[int]:
    """The matrices ``rank`` of ``world`` GPUs owns when whole matrices are dealt out
    round-robin within each size group (matrices of equal element count, in their original
    order; groups in order of first appearance): positions p with p % world == rank."""
    if not 0 <= rank < world:
        raise ValueError("rank must be in [0, world)")
    groups: dict = {}
    for i, (r, c) in enumerate(shapes):
        groups.setdefault(r * c, []).append(i)
    return sorted(i for idx in groups.values() for p, i in enumerate(idx) if p % world == rank)


WORKLOADS = _build()
BY_ID = {wl.cfg_id: wl for wl in WORKLOADS.values()}


def rng(cfg_id: int, kind: int, index: int, step: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_id, kind, index, step])))


def _to_stored(x64: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(dtype)


def weight(wl: Workload, index: int):
    """Initial weights of matrix ``index`` as a CPU torch tensor of the stored dtype."""
    r, c = wl.shapes[index]
    x = rng(wl.cfg_id, KIND_WEIGHT, index, 0).normal(0.0, 0.02, size=(r, c))
    return _to_stored(x, wl.dtype)


def _grad_rng(wl: Workload, index: int, step: int) -> np.random.Generator:
    return rng(wl.cfg_id, KIND_GRAD, index, 0 if wl.reuse_grad else step)


def grad(wl: Workload, index: int, step: int):
    """Gradient of matrix ``index`` at step ``step`` (0-based) as a CPU torch tensor."""
    r, c = wl.shapes[index]
    g = _grad_rng(wl, index, step)
    if wl.iid_t3_entries:
        x = wl.grad_std * g.standard_t(3, size=(r, c))
    elif wl.heavy_tailed_rows:
        t = g.standard_t(3, size=(r, 1))   # the row scales: drawn first (heavy_row_scales)
        z = g.standard_normal(size=(r, c))
        x = wl.grad_std * np.abs(t) * z
    else:
        x = g.normal(0.0, wl.grad_std, size=(r, c))
    return _to_stored(x, wl.dtype)


def heavy_row_scales(wl: Workload, index: int, step: int) -> np.ndarray:
    """|t_i|, the Student-t(3) row scales of a heavy-tailed-rows gradient (rows of matrix
    ``index`` at ``step``), as ``grad`` draws them (its generator's first draw)."""
    if not wl.heavy_tailed_rows:
        raise ValueError(f"{wl.name} has no heavy-tailed rows")
    r, _ = wl.shapes[index]
    return np.abs(_grad_rng(wl, index, step).standard_t(3, size=(r, 1))[:, 0])


def custom(shapes, dtype: str = "bf16", steps: int = 1, grad_std: float = 1e-3,
           cfg_id: int = 100, heavy_tailed_rows: bool = False, reuse_grad: bool = False,
           iid_t3_entries: bool = False) -> Workload:
    """An ad-hoc workload (ragged shapes, mixed sets) with the same seeding scheme."""
    return Workload(f"custom{cfg_id}", cfg_id, tuple(tuple(s) for s in shapes), dtype, steps,
                    grad_std, reuse_grad=reuse_grad, heavy_tailed_rows=heavy_tailed_rows,
                    iid_t3_entries=iid_t3_entries)


def sample_indices(wl: Workload) -> List[int]:
    """A deterministic sample of matrices covering every distinct (rows, cols) of a workload:
    the first, a middle and the last matrix of each shape."""
    out = []
    for shp in dict.fromkeys(wl.shapes):
        idx = [i for i, s in enumerate(wl.shapes) if s == shp]
        for j in sorted({idx[0], idx[len(idx) // 2], idx[-1]}):
            out.append(j)
    return sorted(out)


# ---- non-matrix parameter sets (the Adam half of the optimizer table) ---------------------
#
# The record analysed at lqnn.cn (section 3.3) trains the embedding-like parameters with a
# cautious Adam: the token embedding (tied with the LM head), value-embedding banks and a few
# scalars, with decay multipliers 150 (embed / lm_head) and 0 (scalars). The pages give
# neither the vocabulary nor the number of banks; the sets below use GPT-2's vocabulary of
# 50257 tokens, width 768 and three value-embedding banks, which the pages' 124M model has
# the width of. Value embeddings take the base decay (multiplier 1), since the page's table
# names none for them. Draws use kinds 2 (parameters) and 3 (gradients).

KIND_ADAM_PARAM = 2
KIND_ADAM_GRAD = 3


@dataclass(frozen=True)
class AdamSet:
    name: str
    cfg_id: int
    tensors: Tuple[Tuple[str, Tuple[int, ...], float], ...]   # (label, shape, wd_mul)
    dtype: str                                                  # "bf16" or "f32" for p and g
    steps: int
    param_std: float = 0.02
    grad_std: float = 1e-3

    @property
    def n(self) -> int:
        return len(self.tensors)

    def numel(self, i: int) -> int:
        return int(np.prod(self.tensors[i][1], dtype=np.int64))

    def elements(self) -> int:
        return int(sum(self.numel(i) for i in range(self.n)))


def _adam_sets() -> dict:
    v, d = 50257, 768
    s = {}
    s["gpt2_124m_embed"] = AdamSet(
        "gpt2_124m_embed", 20,
        (("embed", (v, d), 150.0),) + tuple((f"value_embed{k}", (v, d), 1.0) for k in range(3))
        + (("scalars", (64,), 0.0),),
        "bf16", 10)
    s["ragged_small"] = AdamSet(
        "ragged_small", 21,
        (("one", (1,), 1.0), ("odd", (37,), 150.0), ("rows", (5, 129), 1.0),
         ("wide", (3, 1000), 0.0), ("even", (2048,), 150.0), ("vec_tail", (8191,), 1.0),
         ("tile_tail", (3, 4097), 150.0), ("blocks", (70001,), 1.0)),
        "f32", 4, param_std=0.5, grad_std=1.0)
    return s


ADAM_SETS = _adam_sets()


def adam_param(s: AdamSet, index: int):
    """Initial values of tensor ``index`` of an Adam set as a CPU torch tensor."""
    x = rng(s.cfg_id, KIND_ADAM_PARAM, index, 0).normal(0.0, s.param_std,
                                                        size=s.tensors[index][1])
    return _to_stored(x, s.dtype)


def adam_grad(s: AdamSet, index: int, step: int):
    """Gradient of tensor ``index`` at step ``step`` (0-based) as a CPU torch tensor."""
    x = rng(s.cfg_id, KIND_ADAM_GRAD, index, step).normal(0.0, s.grad_std,
                                                          size=s.tensors[index][1])
    return _to_stored(x, s.dtype)


def adam_custom(shapes_wd, dtype: str = "f32", steps: int = 3, cfg_id: int = 200,
                param_std: float = 0.5, grad_std: float = 1.0) -> AdamSet:
    """An ad-hoc Adam set: ``shapes_wd`` is a list of (shape, wd_mul)."""
    return AdamSet(f"adam_custom{cfg_id}", cfg_id,
                   tuple((f"t{i}", tuple(sh), float(w)) for i, (sh, w) in enumerate(shapes_wd)),
                   dtype, steps, param_std=param_std, grad_std=grad_std)
