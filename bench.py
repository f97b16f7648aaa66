"""Throughput of the Muon step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gpt2_124m]

A step is one whole Muon step (momentum, norm, five Newton-Schulz rounds, update) over
every matrix of the workload, on inputs already resident in HBM (weights, fp32 momentum and
two staged gradient batches used alternately). Prints one JSON line:

  value      Muon steps/s over K timed steps (HIP events on the library's stream,
             bracketed by device synchronisation); `repeats`: the median, min and max of
             further timed passes of the same K steps (--repeats, default 5)
  roofline   the dominant kernel kind: algorithmic flops (or bytes) of its launches divided
             by their summed duration, measured with the library's per-launch HIP events in
             a second timed pass of the same K steps (its step time is reported as
             ms_per_step_profiled_pass), against the MI355X peak
  cpu_baseline  the float64 CPU oracle on a bounded sample of the same workload
  next_rows  the cautious-Adam step for the non-matrix parameters of the same model (the
             embedding-shaped set: 4 x 50257 x 768 bf16 + 64 scalars), timed on its own:
             one launch per step, HBM bytes of the algorithm over the launch time; and the
             same Muon step with the per-row energy equaliser switched on (its extra cost)

  mfma_bound the Newton-Schulz products' matrix-core issue bound: each product launch of a
             round replayed with the same grid and MFMAs per wave but no memory traffic
             (libmuon_mfma_loop.so), its time and shader clock; against it, the fraction of
             that bound the products reach

  library_ceiling  what the vendor GEMM library (hipBLASLt, through torch.bmm / torch.matmul)
             reaches on the same box in the same run: the apply products of the workload's
             shape groups as plain batched GEMMs, and one large 8192^3 GEMM; a comparison
             only, nothing of the step runs through it

    python bench.py --adam-only     times only the cautious-Adam step (for profiling it)
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import seeded_inputs as si  # noqa: E402
from orthogonalized_momentum_optimizer_amd import (  # noqa: E402
    MuonPlan, cautious_adam_step, make_adam_config, make_config)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix-core peak
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 vector peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def kind_work(wl, ns_steps=5):
    """Algorithmic work per step of each kernel kind: flops for the products (nominal,
    m <= n: gram 2 m^2 n, poly 2 m^3, apply 2 m^2 n per round), bytes for the elementwise
    kernels (momentum: read G, read+write fp32 M; update: read+write W)."""
    w = {"gram": 0.0, "poly": 0.0, "apply": 0.0, "momentum": 0.0, "update": 0.0, "norm": 0.0,
         "rounds": 0.0}
    esz = 2 if wl.dtype == "bf16" else 4
    for r, c in wl.shapes:
        m, n = min(r, c), max(r, c)
        w["gram"] += ns_steps * 2.0 * m * m * n
        w["poly"] += ns_steps * 2.0 * m ** 3
        w["apply"] += ns_steps * 2.0 * m * m * n
        w["momentum"] += r * c * (esz + 8.0)
        w["update"] += r * c * (2.0 * esz)
    w["rounds"] = w["gram"] + w["poly"] + w["apply"]   # the single-launch rounds
    return w


NS_KINDS = ("gram", "poly", "apply", "rounds")


def shape_groups(wl):
    """The plan's shape groups: (count, mp, np) of the padded wide shapes (rows and cols
    swapped when rows > cols, each rounded up to a multiple of 128)."""
    from collections import Counter
    cnt = Counter()
    for r, c in wl.shapes:
        m, n = min(r, c), max(r, c)
        cnt[(-(-m // 128) * 128, -(-n // 128) * 128)] += 1
    return [(b, mp, np_) for (mp, np_), b in sorted(cnt.items())]


def fused_rounds(groups, ns_steps, cus=256):
    """Whether the library runs these groups' rounds as one persistent launch (its default
    where it applies): bf16, 1-16 rounds, at most 4 groups, each 256-aligned with at least 8
    matrices, a 256-CU device, and at most 8 apply tiles of 256x256 per CU per round."""
    tiles = sum(b * (mp // 256) * (np_ // 256) for b, mp, np_ in groups)
    return (1 <= ns_steps <= 16 and 1 <= len(groups) <= 4 and cus == 256 and
            all(mp % 256 == 0 and np_ % 256 == 0 and b >= 8 for b, mp, np_ in groups) and
            tiles <= 8 * cus)


def product_launches(wl, cus, fused=True, ns_steps=5):
    """Grid, register tile and K steps of the bf16 product launches, as the library launches
    them: with the rounds in one persistent launch (fused_rounds), that launch with its
    K steps dealt evenly over the compute units, group "all" (its entry covers every round);
    otherwise every product launch of one round, group by group (sets whose groups share
    launches are not modelled: returns None). Each entry: (kind, group, blocks, nacc, iters,
    lds): blocks of 256 threads, nacc 32x32 accumulator blocks per wave (16: a 128x128
    register tile, 4: 64x64), iters 32-deep K steps per wave of the busiest block, lds bytes
    per block (which sets the blocks per compute unit)."""
    groups = shape_groups(wl)
    if fused and fused_rounds(groups, ns_steps, cus):
        # one persistent launch, one block per CU, every round's items and tiles dealt evenly
        units = 0
        for b, mp, np_ in groups:
            S = mp // 256
            items = b * S * (S - 1) // 2 + 3 * (b * S // 4) + (b * S) % 4
            units += items * (np_ // 32) + items * (mp // 32)
            units += b * (mp // 256) * (np_ // 256) * (mp // 32)
        return [("rounds", "all", cus, 16, -(-units * ns_steps // cus), 131072)]
    tiles256 = sum(b * -(-mp // 256) * -(-np_ // 256) for b, mp, np_ in groups)
    if len(groups) > 1 and tiles256 < 2 * cus:
        return None
    out = []
    for b, mp, np_ in groups:
        for kind, K in (("gram", np_), ("poly", mp)):
            if mp >= 1024:
                t = -(-mp // 256)
                out.append((kind, (b, mp, np_), b * t * (t + 1) // 2, 16, K // 32, 131072))
                continue
            S = mp // 256
            items = (b * S * (S - 1) // 2 + 3 * (b * S // 4) + (b * S) % 4) if mp % 256 == 0 else 0
            if mp % 256 == 0 and items >= 2 * cus - cus // 8:
                out.append((kind, (b, mp, np_), items, 16, K // 32, 131072))
            else:
                t = mp // 128
                out.append((kind, (b, mp, np_), b * t * (t + 1) // 2, 4, K // 32, 65536))
        tiles = b * -(-mp // 256) * -(-np_ // 256)
        if 2 * tiles <= cus:
            out.append(("apply", (b, mp, np_), 4 * tiles, 4, mp // 32, 65536))
        else:
            per = -(-tiles // cus)
            nb = min(cus, (-(-tiles // per) + 7) // 8 * 8)
            out.append(("apply", (b, mp, np_), nb, 16, per * (mp // 32), 131072))
    return out


def mfma_bound(wl, dev, measured_ns_ms, ns_steps=5, reps=5, fused=True):
    """The matrix-core issue bound of the Newton-Schulz products: every product launch of a
    round (product_launches) replayed by a kernel that issues the same MFMAs per wave on
    the same grid with no memory traffic (libmuon_mfma_loop.so), timed with HIP events, its
    shader clock read from per-block timestamps. The sum over a step is the time the products
    would take if their matrix cores never waited for data at the clock the device then
    holds; its ratio to the measured product time is the fraction of that bound reached."""
    import ctypes
    from orthogonalized_momentum_optimizer_amd import build as b
    launches = product_launches(wl, torch.cuda.get_device_properties(dev).multi_processor_count,
                                fused=fused, ns_steps=ns_steps)
    if launches is None or not os.path.exists(b.PROBE_LIB):
        return None
    lib = ctypes.CDLL(b.PROBE_LIB)
    lib.muon_mfma_loop.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 3 + [
        ctypes.POINTER(ctypes.c_float)]
    lib.muon_mfma_loop.restype = ctypes.c_int
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    rows, total_us = [], 0.0
    for kind, grp, blocks, nacc, iters, lds in launches:
        sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
        stamps = torch.zeros(blocks * 4, dtype=torch.int64, device=dev)
        times = []
        for _ in range(reps + 1):
            t = ctypes.c_float(0.0)
            st = lib.muon_mfma_loop(blocks, nacc, iters, lds, sink.data_ptr(), stamps.data_ptr(),
                                    ctypes.c_void_p(stream.cuda_stream), ctypes.byref(t))
            if st != 0:
                raise RuntimeError(f"muon_mfma_loop failed ({st})")
            times.append(t.value)
        us = sorted(times[1:])[len(times[1:]) // 2]
        sv = stamps.view(blocks, 4).cpu().double()
        cyc = (sv[:, 1] - sv[:, 0]).median().item()
        ghz = ((sv[:, 1] - sv[:, 0]) / (sv[:, 3] - sv[:, 2]) * 0.1).median().item()
        # a 32x32x16 MFMA occupies its SIMD for 32 cycles at the peak rate
        rows.append({"kind": kind,
                     "group": grp if isinstance(grp, str) else f"{grp[0]}x{grp[1]}x{grp[2]}",
                     "blocks": blocks,
                     "tile_per_wave": "128x128" if nacc == 16 else "64x64",
                     "k_steps_per_wave": iters, "us": us, "clock_ghz": ghz,
                     "loop_cycles_per_wave": cyc,
                     "issue_frac": iters * 2 * nacc * 32 / cyc if cyc > 0 else None})
        total_us += us if kind == "rounds" else ns_steps * us
    bound_ms = total_us * 1e-3
    ns_flops = wl.ns_flops_per_step()
    return {"launches": rows, "ns_ms_per_step": bound_ms,
            "ns_frac_of_peak_at_bound": ns_flops / (bound_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "measured_ns_ms_per_step": measured_ns_ms,
            "frac_of_bound_reached": bound_ms / measured_ns_ms if measured_ns_ms else None}


def library_ceiling(wl, dev, apply_tflops, iters=20):
    """hipBLASLt (torch.bmm / torch.matmul, bf16 in, fp32 accumulate, bf16 out) on the apply
    products of the workload's shape groups, X' = B' X with B' (batch x m x m) and X
    (batch x m x n), m <= n, both operands contiguous; and one 8192^3 GEMM, the large-GEMM
    rate of the same box. Random operands; a measurement beside the step, not part of it."""
    groups = {}
    for r, c in wl.shapes:
        m, n = min(r, c), max(r, c)
        groups[(m, n)] = groups.get((m, n), 0) + 1
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    per, tot_ms, tot_fl = {}, 0.0, 0.0
    for (m, n), b in sorted(groups.items()):
        B = torch.randn((b, m, m), device=dev, generator=gen).bfloat16()
        X = torch.randn((b, m, n), device=dev, generator=gen).bfloat16()
        Y = torch.empty((b, m, n), device=dev, dtype=torch.bfloat16)
        ms = timed(lambda: torch.bmm(B, X, out=Y))
        fl = 2.0 * b * m * m * n
        per[f"{b}x{m}x{m} @ {b}x{m}x{n}"] = {"us": 1e3 * ms, "tflops": fl / ms / 1e9}
        tot_ms += ms
        tot_fl += fl
        del B, X, Y
    big = 8192
    P = torch.randn((big, big), device=dev, generator=gen).bfloat16()
    Q = torch.randn((big, big), device=dev, generator=gen).bfloat16()
    R = torch.empty((big, big), device=dev, dtype=torch.bfloat16)
    ms_big = timed(lambda: torch.matmul(P, Q, out=R))
    del P, Q, R
    torch.cuda.empty_cache()
    lib_apply = tot_fl / tot_ms / 1e9
    big_tf = 2.0 * big ** 3 / ms_big / 1e9
    return {"kind": "hipBLASLt via torch.bmm / torch.matmul, bf16, same box and run",
            "apply_shapes": per, "apply_shapes_tflops": lib_apply,
            "gemm_8192_tflops": big_tf, "gemm_8192_frac_of_peak": big_tf / PEAK_BF16_TFLOPS,
            "apply_kernel_tflops": apply_tflops,
            "apply_kernel_over_library_same_shapes": (apply_tflops / lib_apply
                                                      if apply_tflops else None),
            "apply_kernel_over_gemm_8192": apply_tflops / big_tf if apply_tflops else None}


KERNEL_SOURCES = {   # kernel kind -> the source files that define its bf16 kernel
    "apply": ("ns_apply_bf16.hip",), "gram": ("ns_gemm_bf16.hip",),
    "poly": ("ns_gemm_bf16.hip",), "rounds": ("ns_fused_bf16.hip", "ns_quad_item.h"),
    "momentum": ("elementwise.hip",), "update": ("elementwise.hip",),
    "norm": ("elementwise.hip",), "cautious_adam": ("cautious_adam.hip",),
}


def measured_traffic(kind, workload):
    """HBM bytes per launch of a kernel kind, from the rocprofv3 counter summary committed
    under profiles/ (FETCH_SIZE + WRITE_SIZE per dispatch, scaled by a plain copy of known
    size). None when there is no summary or the kernel's sources changed since it was taken
    (the summary holds the SHA-256 of its source files concatenated in KERNEL_SOURCES order)."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}_traffic.md")
    srcs = [os.path.join(ROOT, "orthogonalized_momentum_optimizer_amd", "csrc", f)
            for f in KERNEL_SOURCES.get(kind, ())]
    if not os.path.exists(path) or not srcs or not all(os.path.exists(f) for f in srcs):
        return None
    text = open(path).read()
    m_b = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    m_h = re.search(r"^source_sha256:\s*([0-9a-f]+)", text, re.M)
    if not m_b or not m_h:
        return None
    digest = hashlib.sha256(b"".join(open(f, "rb").read() for f in srcs)).hexdigest()
    if digest != m_h.group(1):
        return None
    return float(m_b.group(1))


def cpu_baseline(wl, budget_s=12.0):
    """The oracle, as it stands, on whole matrices of the workload (one step from zero
    momentum each), in workload order until ``budget_s`` is spent; scaled to one full step
    by nominal Newton-Schulz flops."""
    import numpy as np
    import oracle
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max(int(i.get("num_threads", 1)) for i in infos)
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in infos)
    except Exception:
        cores = os.cpu_count() or 1
    cpu_model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    # only the oracle's own calls are timed: each matrix's inputs are drawn (and upcast to
    # float64, as the oracle does first) before its clock starts
    elapsed, gen_s = 0.0, 0.0
    done_flops, used = 0.0, 0
    for i, (r, c) in enumerate(wl.shapes):
        g0 = time.perf_counter()
        W = si.weight(wl, i).double().numpy()
        G = si.grad(wl, i, 0).double().numpy()
        M = np.zeros((r, c))
        t0 = time.perf_counter()
        gen_s += t0 - g0
        oracle.muon_step(W, M, G)
        elapsed += time.perf_counter() - t0
        m, n = min(r, c), max(r, c)
        done_flops += 5 * (4.0 * m * m * n + 2.0 * m ** 3)
        used = i + 1
        if elapsed > budget_s:
            break
    frac = done_flops / wl.ns_flops_per_step()
    sec_per_step = elapsed / frac
    return {"value": 1.0 / sec_per_step, "unit": "Muon steps/s", "cores": cores,
            "kind": "oracle", "blas": blas, "cpu_model": cpu_model,
            "host_cpus": os.cpu_count(),
            "sample": f"float64 oracle, one step of matrices 0..{used - 1} of {wl.name} "
                      f"({used}/{wl.n} matrices, {frac * 100:.1f}% of the step's nominal flops),"
                      f" scaled to the full step by flops; {elapsed:.1f} s in the oracle "
                      f"(input generation, {gen_s:.1f} s, not timed)"}


def adam_bytes_per_element(pdt="bf16", gdt="bf16"):
    """Algorithmic HBM bytes of one cautious-Adam element: read p, g, m, v; write p, m, v."""
    pe, ge = (2 if pdt == "bf16" else 4), (2 if gdt == "bf16" else 4)
    return 2 * pe + ge + 16


def bench_adam(steps, warmup, dev):
    """Times the cautious-Adam step over the embedding-shaped set of the GPT-2-124M model on
    HBM-resident tensors (parameters and two gradient batches drawn on the GPU from a seeded
    generator; moments zero at the start)."""
    aset = si.ADAM_SETS["gpt2_124m_embed"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(aset.cfg_id)
    numels = [aset.numel(i) for i in range(aset.n)]
    P = [(aset.param_std * torch.randn(n, generator=gen, device=dev)).to(torch.bfloat16)
         for n in numels]
    G = [[(aset.grad_std * torch.randn(n, generator=gen, device=dev)).to(torch.bfloat16)
          for n in numels] for _ in range(2)]
    M = [torch.zeros(n, dtype=torch.float32, device=dev) for n in numels]
    V = [torch.zeros(n, dtype=torch.float32, device=dev) for n in numels]
    muls = [w for _, _, w in aset.tensors]
    lr, betas, eps, wd = 1e-3, (0.9, 0.95), 1e-8, 0.01
    cfgs = [make_adam_config(lr, betas, eps, wd, t + 1) for t in range(warmup + steps)]
    stream = torch.cuda.current_stream()
    for t in range(warmup):
        cautious_adam_step(P, G[t % 2], M, V, cfgs[t], muls)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for t in range(warmup, warmup + steps):
        cautious_adam_step(P, G[t % 2], M, V, cfgs[t], muls)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    elems = aset.elements()
    nbytes = elems * adam_bytes_per_element()
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(f"[bench] cautious Adam: {ms:.4f} ms/step, {gbs:.0f} GB/s", file=sys.stderr,
          flush=True)
    return {"workload": aset.name, "elements": elems,
            "tensors": [f"{lab} {'x'.join(map(str, sh))} wd_mul {w:g}"
                        for lab, sh, w in aset.tensors],
            "dtype": "bf16 params and grads, fp32 moments, fp32 arithmetic",
            "config": {"lr": lr, "betas": list(betas), "eps": eps, "weight_decay": wd},
            "data": "synthetic (seeded GPU draws: N(0,0.02) params, N(0,1e-3) grads, "
                    "2 staged batches)",
            "steps": steps, "warmup": warmup, "ms_per_step": ms,
            "launches_per_step": 1, "value": 1000.0 / ms, "unit": "Adam steps/s",
            "roofline": {"kernel": "cautious_adam", "bound": "hbm", "achieved": gbs,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                         "traffic": measured_traffic("cautious_adam", aset.name),
                         "avg_launch_us": 1e3 * ms,
                         "bytes_per_launch": nbytes}}


def bench_roweq(plan, W, G, M, wl, args, ms_plain):
    """The same Muon step with the per-row energy equaliser on (fp32 row state, zero at the
    start): step time, and the equaliser's own kernels (row sums of O^2 over the bf16 X, then
    per-matrix factors) from the library's per-launch events."""
    dev = W[0].device
    V = [torch.zeros(s[0], dtype=torch.float32, device=dev) for s in wl.shapes]
    cfg = make_config(row_equalize=True)
    stream = torch.cuda.current_stream()
    for t in range(args.warmup):
        plan.step(W, G[t % 2], M, cfg, row_vars=V)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for t in range(args.steps):
        plan.step(W, G[t % 2], M, cfg, row_vars=V)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    out = {"ms_per_step": ms, "steps_per_s": 1000.0 / ms, "ms_over_plain_step": ms - ms_plain,
           "config": {"row_beta": cfg.row_beta, "row_eps": cfg.row_eps}}
    if not args.no_profile:
        plan.set_profiling(True)
        for t in range(args.steps):
            plan.step(W, G[t % 2], M, cfg, row_vars=V)
        torch.cuda.synchronize()
        kms, launches = plan.read_profile()["roweq"]
        plan.set_profiling(False)
        elems = wl.elements()
        out["roweq_kernels_ms_per_step"] = kms / args.steps
        out["roweq_launches_per_step"] = launches / args.steps
        # algorithmic bytes: read O (bf16 X, 2 B/element) once for the row sums
        out["rowsum_read_GBps"] = 2.0 * elems / (kms / args.steps * 1e-3) / 1e9
    print(f"[bench] row equaliser: {ms:.4f} ms/step ({ms - ms_plain:+.4f})", file=sys.stderr,
          flush=True)
    return out


def bench_per_product(wl, W, G, M, cfg, args, dev, stream):
    """The same steps with one launch per product (the shape groups on concurrent streams),
    the path sets take that the single launch does not: step time, and the products' nominal
    flops over their summed kernel times from a pass with per-launch timing (where the groups
    run one after the other)."""
    plan = MuonPlan(wl.shapes, [w.dtype for w in W], [w.dtype for w in W], args.precision, dev,
                    fused=False)
    for t in range(max(args.warmup // 2, 1)):
        plan.step(W, G[t % 2], M, cfg)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for t in range(args.steps):
        plan.step(W, G[t % 2], M, cfg)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    plan.set_profiling(True)
    for t in range(args.steps):
        plan.step(W, G[t % 2], M, cfg)
    torch.cuda.synchronize()
    prof = plan.read_profile()
    plan.close()
    prod_ms = {k: prof[k][0] / args.steps for k in ("gram", "poly", "apply")}
    total = sum(prod_ms.values())
    peak = PEAK_BF16_TFLOPS if args.precision == "bf16" else PEAK_F32_TFLOPS
    frac = wl.ns_flops_per_step() / (total * 1e-3) / 1e12 / peak if total > 0 else None
    print(f"[bench] one launch per product: {ms:.4f} ms/step", file=sys.stderr, flush=True)
    return {"ms_per_step": ms, "value": 1000.0 / ms, "products_ms_per_step": prod_ms,
            "ns_frac_of_peak": frac}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gpt2_124m", choices=sorted(si.WORKLOADS))
    ap.add_argument("--precision", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true")
    ap.add_argument("--repeats", type=int, default=5,
                    help="further timed passes of K steps after the reported one (median/min)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the vendor-library GEMM comparison")
    ap.add_argument("--no-adam", action="store_true", help="skip the cautious-Adam leg")
    ap.add_argument("--no-fused", action="store_true",
                    help="one launch per product instead of all rounds in one launch")
    ap.add_argument("--no-alt", action="store_true",
                    help="skip timing the other path (one launch per product) beside it")
    ap.add_argument("--no-mfma-bound", action="store_true",
                    help="skip the matrix-core issue bound of the products")
    ap.add_argument("--no-roweq", action="store_true", help="skip the row-equaliser leg")
    ap.add_argument("--adam-only", action="store_true",
                    help="time only the cautious-Adam step and print its JSON object")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="before timing, copy 256 MiB device to device once (a plain copy of "
                         "known size for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.adam_only:
        if args.copy_calibration:
            src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
            torch.empty_like(src).copy_(src)
            torch.cuda.synchronize()
            del src
        print(json.dumps(bench_adam(args.steps, args.warmup, dev)), flush=True)
        return
    wl = si.WORKLOADS[args.workload]
    n = wl.n
    print(f"[bench] {wl.name}: {n} matrices, {wl.elements() / 1e6:.1f} M elements, "
          f"generating inputs", file=sys.stderr, flush=True)
    W = [si.weight(wl, i).to(dev) for i in range(n)]
    M = [torch.zeros(s, dtype=torch.float32, device=dev) for s in wl.shapes]
    G = [[si.grad(wl, i, t).to(dev) for i in range(n)] for t in range(2)]
    plan = MuonPlan(wl.shapes, [w.dtype for w in W], [w.dtype for w in W], args.precision, dev,
                    fused=not args.no_fused)
    cfg = make_config()
    stream = torch.cuda.current_stream()
    print(f"[bench] workspace {plan.ws_bytes / 2**20:.1f} MiB; warmup {args.warmup}",
          file=sys.stderr, flush=True)

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for t in range(args.warmup):
        plan.step(W, G[t % 2], M, cfg)
    torch.cuda.synchronize()

    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record(stream)
    for t in range(args.steps):
        plan.step(W, G[t % 2], M, cfg)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = start.elapsed_time(stop) / args.steps
    print(f"[bench] {args.steps} steps: {ms:.4f} ms/step (wall {wall * 1e3 / args.steps:.4f})",
          file=sys.stderr, flush=True)

    reps = []
    for _ in range(args.repeats):
        start.record(stream)
        for t in range(args.steps):
            plan.step(W, G[t % 2], M, cfg)
        stop.record(stream)
        torch.cuda.synchronize()
        reps.append(start.elapsed_time(stop) / args.steps)

    work = kind_work(wl)
    ns_flops = wl.ns_flops_per_step()
    out = {
        "metric": "Muon steps/s on GPT-2-124M matrix set; NS TFLOP/s as % bf16 MFMA peak",
        "value": 1000.0 / ms, "unit": "Muon steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if args.precision == "bf16" else "f32",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1e-3) gradients, 2 staged batches)",
        "config": {"workload": wl.name, "matrices": n,
                   "shapes": sorted({f"{r}x{c}": 0 for r, c in wl.shapes}),
                   "ns_steps": 5, "lr": 0.02, "beta": 0.95, "nesterov": True,
                   "precision": args.precision},
        "ns_tflops_whole_step": ns_flops / (ms * 1e-3) / 1e12,
    }
    if reps:
        srt = sorted(reps)
        out["repeats"] = {"n": len(reps), "steps_each": args.steps,
                          "ms_per_step_median": srt[len(srt) // 2], "ms_per_step_min": srt[0],
                          "ms_per_step_max": srt[-1]}

    if not args.no_profile:
        # a second timed pass of the same K steps with the library's per-launch HIP events
        # (on the launch stream); its own step time shows what the events cost
        plan.set_profiling(True)
        torch.cuda.synchronize()
        start.record(stream)
        for t in range(args.steps):
            plan.step(W, G[t % 2], M, cfg)
        stop.record(stream)
        torch.cuda.synchronize()
        out["ms_per_step_profiled_pass"] = start.elapsed_time(stop) / args.steps
        out["profiled_pass_note"] = (
            "kernel durations come from the per-launch HIP events of this second pass; the "
            "events make the pass itself slower per step (ms_per_step_profiled_pass against "
            "ms_per_step) but each duration spans its own kernel only")
        prof = plan.read_profile()
        plan.set_profiling(False)
        kernels = {}
        for k, (kms, launches) in prof.items():
            per_step = kms / args.steps
            kernels[k] = {"ms_per_step": per_step, "launches_per_step": launches / args.steps,
                          "avg_launch_us": 1e3 * kms / max(launches, 1)}
        gemm_ms = sum(prof[k][0] for k in NS_KINDS) / args.steps
        out["kernels"] = kernels
        out["ns_tflops_kernels"] = ns_flops / (gemm_ms * 1e-3) / 1e12 if gemm_ms > 0 else None
        peak_mm = PEAK_BF16_TFLOPS if args.precision == "bf16" else PEAK_F32_TFLOPS
        out["ns_frac_of_peak"] = (out["ns_tflops_kernels"] or 0) / peak_mm
        # the step's roofline: the nominal Newton-Schulz flops at the bf16 peak plus the
        # elementwise kernels' algorithmic bytes (read G, read and write M and W) at the HBM
        # peak, over the measured step time
        ew_bytes = work["momentum"] + work["update"]
        ns_ms = ns_flops / (peak_mm * 1e12) * 1e3
        ew_ms = ew_bytes / (PEAK_HBM_GBS * 1e9) * 1e3
        out["step_roofline"] = {"ns_ms_at_peak": ns_ms, "elementwise_ms_at_peak": ew_ms,
                                "elementwise_bytes": ew_bytes, "step_ms": ms,
                                "frac": (ns_ms + ew_ms) / ms}
        dom = max(prof, key=lambda k: prof[k][0])
        dms, dl = prof[dom]
        if dom in NS_KINDS:
            ach = work[dom] * args.steps / (dms * 1e-3) / 1e12
            out["roofline"] = {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": peak_mm,
                               "unit": "TFLOP/s", "frac": ach / peak_mm,
                               "traffic": measured_traffic(dom, wl.name),
                               "avg_launch_us": 1e3 * dms / max(dl, 1),
                               "work_per_launch": work[dom] * args.steps / max(dl, 1)}
        else:
            ach = work.get(dom, 0.0) * args.steps / (dms * 1e-3) / 1e9
            out["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": ach,
                               "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                               "traffic": measured_traffic(dom, wl.name),
                               "avg_launch_us": 1e3 * dms / max(dl, 1)}

    if not args.no_mfma_bound and args.precision == "bf16" and "kernels" in out:
        gemm_ms = sum(out["kernels"][k]["ms_per_step"] for k in NS_KINDS)
        out["mfma_bound"] = mfma_bound(wl, dev, gemm_ms, fused=not args.no_fused)

    fused_used = "kernels" in out and out["kernels"].get("rounds", {}).get("launches_per_step", 0) > 0
    if fused_used and not args.no_alt:
        out["one_launch_per_product"] = bench_per_product(wl, W, G, M, cfg, args, dev, stream)

    next_rows = {}
    if not args.no_roweq:
        next_rows["row_equalizer"] = bench_roweq(plan, W, G, M, wl, args, ms)
    plan.close()
    if not args.no_adam:
        del W, M, G
        torch.cuda.empty_cache()
        next_rows["cautious_adam"] = bench_adam(args.steps, args.warmup, dev)
    if next_rows:
        out["next_rows"] = next_rows
    if not args.no_ceiling and args.precision == "bf16":
        apply_tf = None
        if "kernels" in out and out["kernels"]["apply"]["ms_per_step"] > 0:
            apply_tf = work["apply"] / (out["kernels"]["apply"]["ms_per_step"] * 1e-3) / 1e12
        out["library_ceiling"] = library_ceiling(wl, dev, apply_tf)

    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl)
    out["host"] = {"cpu": platform.processor() or platform.machine(),
                   "cpu_count": os.cpu_count(), "torch": torch.__version__,
                   "hip": torch.version.hip,
                   "gpu": torch.cuda.get_device_name(dev)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
