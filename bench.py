#!/usr/bin/env python3
"""Benchmark one optimizer step of the Shampoo block preconditioner on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3]

A step is the whole hot path over one batch of synthetic gradients, with the
inputs already resident in HBM: accumulate (EMA of G G^T and G^T G for every
block), scale (trace, damping, power iteration), inverse 4th roots and
U = X_L G X_R.  The default workload is the 360M-shaped transformer step
(24 layers, hidden 1024, MLP 4096, B = 1024: 288 blocks, 576 factors) with
power-iteration scaling and Newton-DB (k = 10 per pass), all fp32.

Prints one JSON line.  `value` is inverse-4th-root blocks (factors) per
second of whole-step time (with --workload c3-f10, where the roots are
refreshed every 10th step, the roots computed per second over whole
10-step periods; ms_per_step is then the amortised step).  `roofline` reports the dominant kernel (the
Newton-DB pair product) from HIP events recorded around each of its launches
during the timed steps; `cpu_baseline` times the float64 oracle on a bounded
sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F32_MFMA = 157.3     # TFLOP/s, MI355X dense fp32 matrix
PEAK_BF16_MFMA = 2500.0   # TFLOP/s, MI355X dense bf16 (and fp16) matrix
METRIC = "inverse-4th-root blocks/s at B=1024 fp32 + optimizer-step ms; % MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["common.h", "gemm_f32.h", "gemm_bf16.h", "kernels_misc.h", "shampoo.hip"]


def source_digest():
    h = hashlib.sha256()
    for s in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "inverse_root_preconditioning_amd", "csrc", s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def workloads():
    from inverse_root_preconditioning_amd import capi
    from inverse_root_preconditioning_amd import workloads as W
    return {
        "c3": dict(cfg=3, spec=W.MODEL_360M, B=1024, solver="newton", variant=capi.NDB_Z, iters=10,
                   prec=capi.F32, nblocks=None,
                   name="360M-shaped optimizer step: 24 layers, hidden 1024, MLP 4096; B=1024, 288 blocks "
                        "(576 factors); power-iteration scaling r=32 T=20; Newton-DB k=10 per pass "
                        "(second pass Z-chained); fp32"),
        "c3-literal": dict(cfg=3, spec=W.MODEL_360M, B=1024, solver="newton", variant=capi.NDB, iters=10,
                           prec=capi.F32, nblocks=None,
                           name="360M-shaped optimizer step, B=1024, 576 factors, Newton-DB k=10 per pass "
                                "(second pass on Y as on the pages), fp32"),
        "c3-share": dict(cfg=3, spec=W.MODEL_360M, B=1024, solver="newton", variant=capi.NDB_Z, iters=10,
                         prec=capi.F32, nblocks=36,
                         name="one GPU's share of 8 of the 360M-shaped step: 36 blocks (72 factors) of "
                              "1024^2, Newton-DB k=10, fp32"),
        "c3-symp": dict(cfg=3, spec=W.MODEL_360M, B=1024, solver="newton", variant=capi.NDB_Z | capi.SYM_COUPLING,
                        iters=10, prec=capi.F32, nblocks=None,
                        name="360M-shaped optimizer step, B=1024, 576 factors, Newton-DB k=10 (second pass "
                             "Z-chained) with the opt-in symmetric coupling product P = Z Y (not the default: less "
                             "stable on ill-conditioned factors), fp32"),
        "c3-cn": dict(cfg=3, spec=W.MODEL_360M, B=1024, solver="newton", variant=capi.CN, iters=10,
                      prec=capi.F32, nblocks=None,
                      name="360M-shaped optimizer step, B=1024, 576 factors, coupled Newton k=10, fp32"),
        "c3-cn16": dict(cfg=3, spec=W.MODEL_360M, B=1024, solver="newton", variant=capi.CN_F16, iters=10,
                        prec=capi.F32, nblocks=None,
                        name="360M-shaped optimizer step, B=1024, 576 factors, coupled Newton k=10 on fp16 "
                             "operands with fp32 accumulation (accumulate, scale, precondition fp32)"),
        "c3-f10": dict(cfg=3, spec=W.MODEL_360M, B=1024, solver="newton", variant=capi.NDB_Z, iters=10,
                       prec=capi.F32, nblocks=None, update_every=10, steps=10,
                       name="360M-shaped optimizer steps, B=1024, 576 factors, Newton-DB k=10 (second pass "
                            "Z-chained), fp32, roots refreshed every 10 steps and cached in between; timed over "
                            "whole 10-step periods, value counts the roots computed"),
        "c5": dict(cfg=5, spec=W.MODEL_1_3B, B=2048, solver="cheby", variant=capi.NDB, degree=24, iters=0,
                   prec=capi.BF16_IN, nblocks=None,
                   name="1.3B-shaped optimizer step: 24 layers, hidden 2048, MLP 8192; B=2048, 288 blocks "
                        "(576 factors); power-iteration scaling; Chebyshev degree 24 with bf16-input "
                        "MFMA, fp32 accumulate"),
    }


def build_inputs(wl, torch, PL, W):
    grads = W.model_gradients(wl["cfg"], wl["spec"])
    tens = [torch.from_numpy(g).cuda() for g in grads]
    table = PL.BlockTable.from_layers(tens, wl["B"])
    outs = [torch.empty_like(t) for t in tens]
    utable = PL.BlockTable.from_layers(outs, wl["B"])
    if wl["nblocks"] is not None:
        k = wl["nblocks"]
        table = PL.BlockTable(_entries(tens, wl["B"])[:k], wl["B"])
        utable = PL.BlockTable(_entries(outs, wl["B"])[:k], wl["B"])
    return grads, tens, table, outs, utable


def _entries(tensors, B):
    out = []
    for t in tensors:
        m, n = t.shape
        for r0 in range(0, m, B):
            for c0 in range(0, n, B):
                out.append((t, r0, c0, min(B, m - r0), min(B, n - c0)))
    return out


def cpu_baseline(wl, grads, budget_s):
    """The float64 oracle on whole blocks of the same workload until `budget_s`
    of host time is spent (at least one block)."""
    import numpy as np
    from oracle import shampoo_oracle as O
    from inverse_root_preconditioning_amd import capi
    from inverse_root_preconditioning_amd import workloads as W
    B = wl["B"]
    layout = W.block_layout([g.shape for g in grads], B)
    n = len(layout) if wl["nblocks"] is None else wl["nblocks"]
    V0 = W.start_vectors(wl["cfg"], 2, B)  # same work per block; factors 0 and 1's starts reused
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = sum(i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas") or None
    except Exception:
        pass
    method = "ndb" if wl["solver"] == "newton" else "cheby"
    chaining = "Z" if (wl["variant"] & 0xff) == capi.NDB_Z else "Y"
    t0 = time.perf_counter()
    done = 0
    for i in range(n):
        br = layout[i]
        g = O.pad_block(grads[br.weight][br.row0:br.row0 + br.rows, br.col0:br.col0 + br.cols], B)
        O.shampoo_step(np.zeros((B, B)), np.zeros((B, B)), g, 0.95, 0.05, 1e-12, "power", V0[0], V0[1],
                       method, steps=20, iters=wl.get("iters", 10), degree=wl.get("degree", 24),
                       chaining=chaining)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    cores = threads or len(os.sched_getaffinity(0))
    return {"value": 2 * done / dt, "unit": "blocks/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {n} blocks ({2 * done} factors) of the same workload through the float64 "
                      f"oracle (accumulate, power-iteration scale, {method} root, precondition) in {dt:.1f} s"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 5; 10 for c3-f10)")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="c3",
                    choices=["c3", "c3-literal", "c3-share", "c3-symp", "c3-cn", "c3-cn16", "c3-f10", "c5"])
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (reference kernel for the HBM byte counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this implementation runs on one GPU only (the multi-GPU sharding is a design, "
              "not built); run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    from inverse_root_preconditioning_amd import capi
    from inverse_root_preconditioning_amd import pipeline as PL
    from inverse_root_preconditioning_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    capi.load()
    wl = workloads()[args.workload]
    if args.steps is None:
        args.steps = wl.get("steps", 5)
    every = wl.get("update_every", 1)
    refreshes = -(-args.steps // every)  # root refreshes in the timed steps (the first one is a refresh)
    B = wl["B"]
    grads, tens, table, outs, utable = build_inputs(wl, torch, PL, W)
    n = table.n
    nf = 2 * n
    cfg = PL.StepConfig(B=B, beta=0.95, eps_rel=1e-12, solver=wl["solver"], variant=wl["variant"],
                        iters=wl.get("iters", 10) or 10, degree=wl.get("degree", 24), prec=wl["prec"],
                        update_every=every)
    state = PL.ShampooBlocks(cfg, n)
    state.set_start_vectors(torch.from_numpy(W.start_vectors(wl["cfg"], nf, B)).cuda())
    stream = torch.cuda.current_stream()

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        state.step(table, utable)
    torch.cuda.synchronize()

    # Per-stage split (one untimed step with events between the stages).
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    ev[0].record()
    PL.accumulate(table, state.factors, cfg.beta, 1 - cfg.beta, cfg.prec, state.ws["acc"])
    ev[1].record()
    PL.scale_power(state.factors, cfg.eps_rel, cfg.scale_mode, state.v0, cfg.pi_steps, cfg.safety, state.scale,
                   state.status, state.ws["scale"])
    ev[2].record()
    if cfg.solver == "newton":
        PL.invroot_newton(state.factors, state.scale, cfg.p, cfg.variant, cfg.iters, state.roots, state.status,
                          None, state.ws["root"])
    else:
        PL.invroot_cheby(state.factors, state.scale, cfg.p, cfg.degree, cfg.interval_eps, cfg.prec, state.roots,
                         state.status, state.ws["root"])
    ev[3].record()
    PL.precondition(state.roots, table, utable, cfg.prec, state.ws["pre"])
    ev[4].record()
    torch.cuda.synchronize()
    stages = {k: ev[i].elapsed_time(ev[i + 1]) for i, k in
              enumerate(["accumulate", "scale", "invroot", "precondition"])}
    # Grafted parameter update (reported beside the step, not part of it).
    params = [t.clone() for t in tens]
    moms = [torch.zeros_like(t) for t in tens]
    vels = [torch.zeros_like(t) for t in tens]
    gtabs = [table, utable] + [PL.BlockTable(_entries(ts, B)[:n], B) for ts in (params, moms, vels)]
    PL.graft_update(*gtabs, 1e-3, 0.9, 0.95, 1e-8, 1)
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    PL.graft_update(*gtabs, 1e-3, 0.9, 0.95, 1e-8, 2)
    g1.record()
    torch.cuda.synchronize()
    graft_ms = g0.elapsed_time(g1)
    del params, moms, vels, gtabs

    # Timing hook on the dominant kernel during the timed steps.
    # Algorithmic flops of one product: 2 B^3 in full; a symmetric product
    # (the default for these launches) needs only its upper triangle with the
    # diagonal, B (B + 1) / 2 entries of 2 B flops each.
    sym_product = float(B) * B * (B + 1)
    # MFMA work a symmetric fp32 product executes: the off-diagonal upper tiles
    # in full and, of each diagonal tile, the 32 x 32 blocks its active waves
    # compute (256 tiles: 9/16 of the tile; 128 tiles: 10/16; 64 tiles: 3/4).
    edge, diag_frac = (256, 9 / 16) if B % 256 == 0 else (128, 10 / 16) if B % 128 == 0 else (64, 3 / 4)
    tiles = B // edge
    executed = 2.0 * B ** 3 * (tiles * (tiles - 1) / 2 + tiles * diag_frac) / tiles ** 2
    f32_kernel = "gemm_f32_big_kernel" if edge == 256 else "gemm_f32_kernel"
    base_variant = cfg.variant & 0xff  # without the modifier bits
    if cfg.solver == "newton" and base_variant in (capi.CN, capi.CN_F16):
        family, per_step = capi.TIME_CN_M, cfg.iters - 1
        flops_per_launch = nf * 2.0 * B ** 3
        mfma_flops = flops_per_launch
        half = base_variant == capi.CN_F16
        peak = PEAK_BF16_MFMA if half else PEAK_F32_MFMA
        h16_cn = "gemm_h16_big_kernel<EpiCnM, fp16, 8 waves>" if B % 256 == 0 else "gemm_h16_nt_kernel<EpiCnM, fp16>"
        f32_cn = "gemm_f32_big_kernel<EpiCnM>" if B % 256 == 0 else "gemm_f32_kernel<EpiCnM>"
        kname = (h16_cn if half else f32_cn) + \
            " (coupled Newton C^p M, one full product per factor)"
    elif cfg.solver == "newton":
        family, per_step = capi.TIME_NDB_PAIR, 2 * (cfg.iters - 2)
        flops_per_launch = 2 * nf * sym_product
        mfma_flops = 2 * nf * executed
        peak, kname = PEAK_F32_MFMA, (f32_kernel + "<EpiPair> (Newton-DB Y E and E Z, 2 symmetric products "
                                      "per factor, upper tiles)")
    else:
        family, per_step = capi.TIME_CLENSHAW, cfg.degree - 1
        flops_per_launch = nf * sym_product
        mfma_flops = nf * executed
        bf = cfg.prec == capi.BF16_IN
        peak = PEAK_BF16_MFMA if bf else PEAK_F32_MFMA
        if bf and B % 256 == 0:
            # 4 x 2 waves of 64 x 128; a diagonal tile computes its 36 upper 32 x 32 blocks (9/16)
            h16_kernel = "gemm_h16_big_kernel<EpiClenshaw, bf16, 8 waves>"
        else:
            h16_kernel = "gemm_h16_nt_kernel<EpiClenshaw, bf16>"
        kname = (h16_kernel if bf else f32_kernel + "<EpiClenshaw>") + \
            " (one symmetric Clenshaw product per factor, upper tiles)"
    cap = max(1, per_step * refreshes)
    kev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * cap)]
    for e in kev:
        e.record(stream)  # materialise the underlying HIP events
    torch.cuda.synchronize()
    handles = (ctypes.c_void_p * (2 * cap))(*[e.cuda_event for e in kev])
    capi.check(capi.shampoo_timing_hook(family, ctypes.addressof(handles), cap), "timing hook")

    state.t = 0  # the timed steps start with a root refresh
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        state.step(table, utable)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    recorded = capi.shampoo_timing_count()
    capi.shampoo_timing_hook(capi.TIME_OFF, None, 0)
    durs = [kev[2 * i].elapsed_time(kev[2 * i + 1]) for i in range(recorded)]

    status = state.status.cpu()
    elapsed = t1 - t0
    ms_step = 1e3 * elapsed / args.steps
    value = nf * refreshes / elapsed
    avg_ms = sum(durs) / len(durs) if durs else float("nan")
    achieved = flops_per_launch / (avg_ms * 1e-3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        rec = tr.get(args.workload)
        if rec and rec.get("source_digest") == source_digest():
            traffic = rec.get("bytes_per_launch")
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16-in/f32" if cfg.prec == capi.BF16_IN else
                  "f16-in/f32" if (cfg.variant & 0xff) == capi.CN_F16 and cfg.solver == "newton" else "f32"),
        "data": "synthetic N(0, 0.02^2) gradients of the workload's weight shapes, seeded",
        "config": dict({"workload": wl["name"], "B": B, "blocks": n, "factors": nf},
                       **({"update_every": every} if every > 1 else {})),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": kname, "launches_timed": recorded, "avg_launch_ms": round(avg_ms, 4),
                     "flops_per_launch": flops_per_launch,
                     "mfma_tflops_executed": round(mfma_flops / (avg_ms * 1e-3) / 1e12, 2)},
        "stages_ms": {k: round(v, 3) for k, v in stages.items()},
        "graft_update_ms": round(graft_ms, 3),
        "invroot_blocks_per_s": round(nf / (stages["invroot"] * 1e-3), 2),
        "status_nonzero_factors": int((status != 0).sum()),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, grads, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
