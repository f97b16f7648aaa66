"""The Muon step at the plan's maximum sizes (rows, cols <= 32768, rows * cols = 2^28), checked
on sampled elements against values the oracle computes exactly at any size.

The gradients have orthogonal rows (or columns): G = diag(r) H, H rows of the Sylvester
Hadamard matrix (entries +-1), r a few distinct row scales. Every entry of a row has the same
magnitude, so the bf16 gradient is exactly of this form, and X0 = U / ||U||_F has the
singular values x_i = r_i / ||r||_2 with singular vectors e_i and H_i / sqrt(n). The
iteration acts on each singular value alone, so O_ij = p5(x_i) H_ij / sqrt(n), with
p5(x) the oracle's five rounds on the 1x1 matrix [x] (oracle.newton_schulz on a diagonal
of the distinct x values). With W0 = 0 the update is W1 = bf16(-lr O).
"""
import numpy as np
import pytest
import torch

import oracle
from orthogonalized_momentum_optimizer_amd import MuonPlan, make_config

pytestmark = pytest.mark.gpu

LEVELS = np.array([1.0, 0.8, 0.55, 0.35, 0.2, 0.12, 0.07, 0.04])   # row scales, cycled


def dev():
    return torch.device("cuda", 0)


def hadamard_sign(i: np.ndarray, j: np.ndarray) -> np.ndarray:
    """(-1)^popcount(i & j) for int64 arrays (the Sylvester Hadamard matrix)."""
    x = np.bitwise_and(i, j)
    par = np.zeros_like(x)
    while np.any(x):
        par ^= x & 1
        x >>= 1
    return 1 - 2 * par


def hadamard_block(r0: int, rows: int, n: int) -> torch.Tensor:
    """Rows r0..r0+rows-1 of the order-n Sylvester Hadamard matrix, +-1, on the GPU."""
    i = torch.arange(r0, r0 + rows, device=dev(), dtype=torch.int32)[:, None]
    j = torch.arange(n, device=dev(), dtype=torch.int32)[None, :]
    x = i & j
    for sh in (16, 8, 4, 2, 1):
        x = x ^ (x >> sh)
    return (1 - 2 * (x & 1)).to(torch.float32)


def make_grad(rows: int, cols: int, levels_idx: np.ndarray) -> torch.Tensor:
    """bf16 gradient with orthogonal rows (rows <= cols) or columns (rows > cols)."""
    m, n = min(rows, cols), max(rows, cols)
    scale = torch.tensor(LEVELS[levels_idx] / np.sqrt(n), dtype=torch.float32, device=dev())
    G = torch.empty(m, n, dtype=torch.bfloat16, device=dev())
    for r0 in range(0, m, 1024):
        k = min(1024, m - r0)
        G[r0:r0 + k] = (hadamard_block(r0, k, n) * scale[r0:r0 + k, None]).to(torch.bfloat16)
    return G if rows <= cols else G.t().contiguous()


def test_maximum_sizes_closed_form():
    shapes = [(16384, 16384), (8192, 32768), (32768, 8192), (1, 32768), (32768, 1)]
    print(f"[maxsize] {shapes}", flush=True)
    plan = MuonPlan(shapes, [torch.bfloat16] * 5, [torch.bfloat16] * 5, "bf16", dev())
    idx = [np.arange(min(s)) % len(LEVELS) for s in shapes]
    G = [make_grad(r, c, k) for (r, c), k in zip(shapes, idx)]
    W = [torch.zeros(s, dtype=torch.bfloat16, device=dev()) for s in shapes]
    M = [torch.zeros(s, dtype=torch.float32, device=dev()) for s in shapes]
    O = [torch.empty(s, dtype=torch.float32, device=dev()) for s in shapes]
    cfg = make_config()
    plan.step(W, G, M, cfg, outs=O)
    torch.cuda.synchronize()
    print("[maxsize] step done", flush=True)
    rng = np.random.Generator(np.random.PCG64(77))
    for q, (rows, cols) in enumerate(shapes):
        m, n = min(rows, cols), max(rows, cols)
        # the bf16 row scales the gradient really holds, and the singular values of X0
        r_store = np.array([float(torch.tensor(LEVELS[k] / np.sqrt(n)).to(torch.bfloat16))
                            for k in range(len(LEVELS))])
        r_rows = r_store[idx[q]] * np.sqrt(n)
        x_levels = r_store * np.sqrt(n) / np.sqrt(np.sum(r_rows ** 2))
        p5 = np.diag(oracle.newton_schulz(np.diag(x_levels), 5))
        # sampled elements: corners, the first and last rows and columns, random ones
        ii = np.concatenate([rng.integers(0, rows, 40000), [0, rows - 1, 0, rows - 1],
                             np.zeros(64, np.int64), np.full(64, rows - 1)])
        jj = np.concatenate([rng.integers(0, cols, 40000), [0, 0, cols - 1, cols - 1],
                             rng.integers(0, cols, 128)])
        a, b = (ii, jj) if rows <= cols else (jj, ii)          # (singular index, H column)
        expect = p5[idx[q][a]] * hadamard_sign(a.astype(np.int64), b.astype(np.int64)) / np.sqrt(n)
        sel = torch.tensor(ii * cols + jj, dtype=torch.long, device=dev())
        got = O[q].reshape(-1)[sel].double().cpu().numpy()
        err = np.sqrt(np.mean((got - expect) ** 2) / np.mean(expect ** 2))
        print(f"[maxsize] {rows}x{cols}: sampled relative error {err:.3e}", flush=True)
        assert err <= 3e-2, f"{rows}x{cols}: sampled O error {err:.3e}"
        w = W[q].reshape(-1)[sel]
        w_expect = (-cfg.lr * O[q].reshape(-1)[sel]).to(torch.bfloat16)
        assert torch.equal(w, w_expect), f"{rows}x{cols}: W != bf16(-lr O)"
    plan.close()
