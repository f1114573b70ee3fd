#!/usr/bin/env python3
"""Benchmark one optimizer step of the Shampoo block preconditioner on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3]

A step is the whole hot path over one batch of synthetic input, with the
inputs already resident in HBM.  For the gradient workloads (c2, c3, c5 and
their variants) that is accumulate (EMA of G G^T and G^T G for every block),
scale (trace, damping, power iteration), inverse 4th roots and
U = X_L G X_R.  For the workloads whose inputs are the SPD factors themselves
(c1: 8 factors of 64^2, c4: 64 ill-conditioned factors of 512^2) it is scale
and inverse roots.  The default workload is the 360M-shaped transformer step
(24 layers, hidden 1024, MLP 4096, B = 1024: 288 blocks, 576 factors) with
power-iteration scaling and Newton-DB (k = 10 per pass), all fp32.

Prints one JSON line.  `value` is inverse-4th-root blocks (factor roots) per
second of whole-step time (with --workload c3-f10, where the roots are
refreshed every 10th step, the roots computed per second over whole 10-step
periods; ms_per_step is then the amortised step).  Every launch of the
hooked kernel families (the Newton-DB pair and coupling products, the
Clenshaw product, coupled Newton's C^p M) during the timed steps is bracketed
by HIP events on its own stream; `kernels` lists each family's average launch
time, its rate in TFLOP/s and GB/s of algorithmic work, and its bound (the
lower roofline at its arithmetic intensity); `roofline` is the family that
took the most time.
`cpu_baseline` times the float64 oracle on a bounded sample of the same
workload on the host cores.
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
PEAK_HBM = 8000.0         # GB/s, MI355X HBM3E
METRIC = "inverse-4th-root blocks/s at B=1024 fp32 + optimizer-step ms; % MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# Device sources of each hooked kernel family: stored HBM counters are used
# only while these hash to the digest recorded with them.
F32_SOURCES = ["common.h", "gemm_f32.h"]
H16_SOURCES = ["common.h", "gemm_f32.h", "gemm_bf16.h"]


ALL_SOURCES = ["common.h", "gemm_f32.h", "gemm_bf16.h", "kernels_misc.h", "shampoo.hip"]


def env_info():
    """Software and device the line was measured with (the box has no git checkout, so the library
    sources are identified by their digest)."""
    import torch
    props = torch.cuda.get_device_properties(0)
    return {"hip": torch.version.hip, "torch": torch.__version__, "gpu": props.name,
            "arch": getattr(props, "gcnArchName", None), "compute_units": props.multi_processor_count,
            "library_sources_digest": source_digest(ALL_SOURCES),
            "seeds": "numpy PCG64(SeedSequence([config, tag, index...])), drawn in float64, rounded once to fp32"}


def source_digest(files):
    h = hashlib.sha256()
    for s in files:
        with open(os.path.join(ROOT, "inverse_root_preconditioning_amd", "csrc", s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def workloads():
    from inverse_root_preconditioning_amd import capi
    from inverse_root_preconditioning_amd import workloads as W
    m360 = dict(cfg=3, kind="model", spec=W.MODEL_360M, B=1024, solver="newton", iters=10, prec=capi.F32,
                nblocks=None, eps_rel=1e-12)
    return {
        "c1": dict(cfg=1, kind="factors", B=64, solver="newton", variant=capi.CN, iters=12, prec=capi.F32,
                   eps_rel=0.0, scale=capi.SCALE_POWER,
                   name="8 SPD blocks 64x64 fp32 (A = G G^T/128 + 1e-6 I, G ~ N(0,1) 64x128, seed 0): "
                        "power-iteration scaling (20 steps) and coupled Newton k=12"),
        "c2": dict(cfg=2, kind="stream", B=256, solver="newton", variant=capi.NDB_Z, iters=10, prec=capi.F32,
                   eps_rel=1e-12,
                   name="one 1024x1024 linear-layer gradient per step, N(0, 0.02^2), 5 gradients in turn: 16 "
                        "blocks of 256^2 (32 factors), EMA beta2=0.95, eps=1e-12 tr/B, power-iteration "
                        "scaling, Newton-DB k=10 per pass (second pass Z-chained), fp32"),
        "c2-literal": dict(cfg=2, kind="stream", B=256, solver="newton", variant=capi.NDB, iters=10,
                           prec=capi.F32, eps_rel=1e-12,
                           name="config 2 (16 blocks of 256^2 per 1024x1024 gradient) with Newton-DB k=10, "
                                "second pass on Y as on the pages, fp32"),
        "c3": dict(m360, variant=capi.NDB_Z,
                   name="360M-shaped optimizer step: 24 layers, hidden 1024, MLP 4096; B=1024, 288 blocks "
                        "(576 factors); power-iteration scaling r=32 T=20; Newton-DB k=10 per pass "
                        "(second pass Z-chained); fp32"),
        "c3-literal": dict(m360, variant=capi.NDB,
                           name="360M-shaped optimizer step, B=1024, 576 factors, Newton-DB k=10 per pass "
                                "(second pass on Y as on the pages), fp32"),
        "c3-share": dict(m360, variant=capi.NDB_Z, nblocks=36,
                         name="one GPU's share of 8 of the 360M-shaped step: 36 blocks (72 factors) of "
                              "1024^2, Newton-DB k=10, fp32"),
        "c3-symp": dict(m360, variant=capi.NDB_Z | capi.SYM_COUPLING,
                        name="360M-shaped optimizer step, B=1024, 576 factors, Newton-DB k=10 (second pass "
                             "Z-chained) with the opt-in symmetric coupling product P = Z Y (not the default: less "
                             "stable on ill-conditioned factors), fp32"),
        "c3-cn": dict(m360, variant=capi.CN,
                      name="360M-shaped optimizer step, B=1024, 576 factors, coupled Newton k=10, fp32"),
        "c3-cn16": dict(m360, variant=capi.CN_F16,
                        name="360M-shaped optimizer step, B=1024, 576 factors, coupled Newton k=10 on fp16 "
                             "operands with fp32 accumulation (accumulate, scale, precondition fp32)"),
        "c3-f10": dict(m360, variant=capi.NDB_Z, update_every=10, steps=10,
                       name="360M-shaped optimizer steps, B=1024, 576 factors, Newton-DB k=10 (second pass "
                            "Z-chained), fp32, roots refreshed every 10 steps and cached in between; timed over "
                            "whole 10-step periods, value counts the roots computed"),
        "c4": dict(cfg=4, kind="factors", B=512, solver="newton", variant=capi.NDB_Z, iters=10, prec=capi.F32,
                   eps_rel=0.0, scale=capi.SCALE_POWER,
                   name="64 SPD blocks 512x512 fp32, A = Q diag(lambda) Q^T, Q Haar, lambda log-uniform in "
                        "[1e-8, 1]: power-iteration scaling, Newton-DB k=10 per pass (second pass Z-chained)"),
        "c4-literal": dict(cfg=4, kind="factors", B=512, solver="newton", variant=capi.NDB, iters=7,
                           prec=capi.F32, eps_rel=0.0, scale=capi.SCALE_POWER,
                           name="config 4 (64 SPD blocks 512^2, lambda in [1e-8, 1]): power-iteration scaling, "
                                "Newton-DB k=7 per pass, second pass on Y as on the pages (the deepest cell of "
                                "that chaining fp32 can match)"),
        "c4-frob": dict(cfg=4, kind="factors", B=512, solver="newton", variant=capi.NDB_Z, iters=10,
                        prec=capi.F32, eps_rel=0.0, scale=capi.SCALE_FROBENIUS,
                        name="config 4 (64 SPD blocks 512^2, lambda in [1e-8, 1]): Frobenius scaling, "
                             "Newton-DB k=10 per pass (second pass Z-chained)"),
        "c4-cheby16": dict(cfg=4, kind="factors", B=512, solver="cheby", degree=16, prec=capi.F32, eps_rel=0.0,
                           scale=capi.SCALE_POWER,
                           name="config 4 (64 SPD blocks 512^2, lambda in [1e-8, 1]): power-iteration scaling, "
                                "Chebyshev degree 16 (Clenshaw), fp32"),
        "c4-cheby32": dict(cfg=4, kind="factors", B=512, solver="cheby", degree=32, prec=capi.F32, eps_rel=0.0,
                           scale=capi.SCALE_POWER,
                           name="config 4 (64 SPD blocks 512^2, lambda in [1e-8, 1]): power-iteration scaling, "
                                "Chebyshev degree 32 (Clenshaw), fp32"),
        "c5": dict(cfg=5, kind="model", spec=W.MODEL_1_3B, B=2048, solver="cheby", degree=24, prec=capi.BF16_IN,
                   nblocks=None, eps_rel=1e-12,
                   name="1.3B-shaped optimizer step: 24 layers, hidden 2048, MLP 8192; B=2048, 288 blocks "
                        "(576 factors); power-iteration scaling; Chebyshev degree 24 with bf16-input "
                        "MFMA, fp32 accumulate"),
    }


def _entries(tensors, B):
    out = []
    for t in tensors:
        m, n = t.shape
        for r0 in range(0, m, B):
            for c0 in range(0, n, B):
                out.append((t, r0, c0, min(B, m - r0), min(B, n - c0)))
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return sum(i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas") or None
    except Exception:
        return None


def cpu_baseline(wl, inputs, budget_s):
    """The float64 oracle on whole blocks (or factors) of the same workload
    until `budget_s` of host time is spent (at least one)."""
    import numpy as np
    from oracle import shampoo_oracle as O
    from inverse_root_preconditioning_amd import capi
    from inverse_root_preconditioning_amd import workloads as W
    B = wl["B"]
    chaining = "Z" if (wl.get("variant", 0) & 0xff) == capi.NDB_Z else "Y"
    method = "cheby" if wl["solver"] == "cheby" else ("cn" if (wl["variant"] & 0xff) in (capi.CN, capi.CN_F16)
                                                      else "ndb")
    kw = dict(iters=wl.get("iters", 10), degree=wl.get("degree", 24), chaining=chaining)
    t0 = time.perf_counter()
    done = 0
    if wl["kind"] == "factors":
        A = inputs
        nf = A.shape[0]
        V0 = W.start_vectors(wl["cfg"], nf, B)
        mode = "power" if wl["scale"] == capi.SCALE_POWER else "frobenius"
        while True:
            i = done % nf
            sc = O.scale_factor(A[i], wl["eps_rel"], mode, V0[i], 20, 2.0)
            O.invroot(A[i], sc, method, **kw)
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        what = f"{done} factor roots ({done / nf:.2f} passes over the {nf} factors)"
        value = done / (time.perf_counter() - t0)
    else:
        grads = inputs
        layout = W.block_layout([g.shape for g in grads], B)
        n = len(layout) if wl.get("nblocks") is None else wl["nblocks"]
        V0 = W.start_vectors(wl["cfg"], 2, B)  # same work per block; factors 0 and 1's starts reused
        while True:
            br = layout[done % n]
            g = O.pad_block(grads[br.weight][br.row0:br.row0 + br.rows, br.col0:br.col0 + br.cols], B)
            O.shampoo_step(np.zeros((B, B)), np.zeros((B, B)), g, 0.95, 0.05, wl["eps_rel"], "power", V0[0], V0[1],
                           method, steps=20, **kw)
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        what = (f"{done} blocks ({2 * done} factor roots), cycling over the {n} blocks of one step, each "
                f"through accumulate, power-iteration scale, the {method} root and precondition")
        value = 2 * done / (time.perf_counter() - t0)
    dt = time.perf_counter() - t0
    cores = blas_threads() or len(os.sched_getaffinity(0))
    return {"value": round(value, 4), "unit": "blocks/s", "cores": cores, "kind": "oracle", "cpu": cpu_model(),
            "sample": f"float64 numpy oracle (matrix products through the host BLAS) on {what}, {dt:.1f} s"}


def family_sources(fam, wl, capi):
    half = wl["prec"] == capi.BF16_IN or (wl.get("solver") == "newton" and (wl.get("variant", 0) & 0xff) == capi.CN_F16)
    return H16_SOURCES if half and fam in (capi.TIME_CLENSHAW, capi.TIME_CN_M) else F32_SOURCES


def family_info(fam, wl, B, nf, capi):
    """(kernel name, algorithmic flops per launch, algorithmic HBM bytes per
    launch, MFMA peak TFLOP/s) of a hooked family.  Bytes count every operand
    read once and every output written once, per factor:
      Newton-DB Y E and E Z: read Y, E, Z, write Y, Z (fp32)          20 B^2
      Newton-DB P = Z Y:     read Z, Y, write E                        12 B^2
      Clenshaw, fp32:        read A_s, b1 (operands), b1 and b2 at the
                             upper entries, write b in full            16 B^2
      Clenshaw, bf16 input:  read the bf16 A_s^T and b1 copies, b1 and b2
                             (fp32) at the upper entries, write b (fp32)
                             at the upper entries and its bf16 copy    12 B^2
                             (10 B^2 with B a multiple of 256, where the
                             bf16 b1 and b copies are kept on and above
                             the diagonal, counted as a triangle: B^2 each)
      coupled Newton C^p M:  read C^p, M, write M, C: fp32 16 B^2, fp16 8 B^2
                             (fp16 with B a multiple of 256 and symmetric
                             products: C^p kept on and above the diagonal,
                             read as a triangle, 7 B^2)"""
    sym = float(B) * B * (B + 1)   # one symmetric product: upper triangle with the diagonal
    full = 2.0 * B ** 3
    b2 = float(B) * B
    v = wl.get("variant", 0)
    full_all = bool(v & capi.FULL_PRODUCTS)
    sym_c = bool(v & capi.SYM_COUPLING) and not full_all
    big = B % 256 == 0
    f32k = "gemm_f32_big_kernel" if big else "gemm_f32_kernel"
    if fam == capi.TIME_NDB_PAIR:
        return (f32k + "<EpiPair> (Newton-DB Y E and E Z, 2 symmetric products per factor, upper tiles)",
                nf * 2 * (full if full_all else sym), nf * 20 * b2, PEAK_F32_MFMA)
    if fam == capi.TIME_NDB_P:
        return (f32k + "<EpiNdbE> (Newton-DB P = Z Y with E = (3I - P)/2 and the residual, "
                + ("upper tiles" if sym_c else "full product") + ")",
                nf * (sym if sym_c else full), nf * 12 * b2, PEAK_F32_MFMA)
    if fam == capi.TIME_CLENSHAW:
        bf = wl["prec"] == capi.BF16_IN
        if bf:
            k = "gemm_h16_big_kernel<EpiClenshaw, bf16, 8 waves>" if big else "gemm_h16_nt_kernel<EpiClenshaw, bf16>"
        else:
            k = f32k + "<EpiClenshaw>"
        upper16 = bf and big and not full_all
        return (k + " (one symmetric Clenshaw product per factor, upper tiles)", nf * (full if full_all else sym),
                nf * ((10 if upper16 else 12) if bf else 16) * b2, PEAK_BF16_MFMA if bf else PEAK_F32_MFMA)
    half = (v & 0xff) == capi.CN_F16
    if half:
        k = "gemm_h16_big_kernel<EpiCnM, fp16, 8 waves>" if big else "gemm_h16_nt_kernel<EpiCnM, fp16>"
    else:
        k = f32k + "<EpiCnM>"
    p = wl.get("p", 4)
    upper16 = half and big and not full_all and p >= 2  # p = 1: C^p is C, kept in full
    return (k + " (coupled Newton C^p M with C = ((p+1)I - M)/p and the residual, "
            + ("upper tiles" if sym_c else "full product") + ")",
            nf * (sym if sym_c else full), nf * ((7 if upper16 else 8) if half else 16) * b2,
            PEAK_BF16_MFMA if half else PEAK_F32_MFMA)


FAMILY_KEYS = {1: "ndb_pair", 2: "ndb_p", 4: "clenshaw", 8: "cn_m"}


def stage_rates(wl, cfg, B, n, nf, stages, capi):
    """Algorithmic rates of the stages around the roots, from the stage-split
    step (HIP events between the stages on the step's stream), each against
    the lower roofline at its arithmetic intensity:
      accumulate:   two symmetric products per block, B^2 (B + 1) flops each;
                    20 B^2 bytes per block (G read, L and R read and written)
      scale:        power iteration, T + 1 products F V of r columns per
                    factor: 2 B^2 r (T + 1) flops and 4 B^2 (T + 1) bytes (F
                    read each round; fp32 MFMA); Frobenius: F read once
      precondition: two full products per block, 4 B^3 flops; 16 B^2 bytes
                    per block (X_L, X_R and G read, U written)
    The products run on bf16-input MFMA for bf16-input workloads, else fp32."""
    b2 = float(B) * B
    mm = PEAK_BF16_MFMA if wl["prec"] == capi.BF16_IN else PEAK_F32_MFMA
    if cfg.scale_mode == capi.SCALE_POWER:
        t1 = cfg.pi_steps + 1
        sc = (nf * 2 * b2 * cfg.pi_starts * t1, nf * 4 * b2 * t1, PEAK_F32_MFMA)
    else:
        sc = (nf * 2 * b2, nf * 4 * b2, PEAK_F32_MFMA)
    work = {"accumulate": (n * 2 * b2 * (B + 1), n * 20 * b2, mm), "scale": sc,
            "precondition": (n * 4.0 * B ** 3, n * 16 * b2, mm)}
    out = {}
    for name, (flops, nbytes, peak) in work.items():
        ms = stages.get(name)
        if not ms:
            continue
        tflops, gbs = flops / (ms * 1e-3) / 1e12, nbytes / (ms * 1e-3) / 1e9
        hbm = flops / nbytes < peak * 1e12 / (PEAK_HBM * 1e9)
        out[name] = {"ms": round(ms, 3), "tflops": round(tflops, 2), "gbs": round(gbs, 1),
                     "bound": "hbm" if hbm else "mfma", "peak": PEAK_HBM if hbm else peak,
                     "frac": round(gbs / PEAK_HBM if hbm else tflops / peak, 4),
                     "flops": flops, "bytes": nbytes}
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 5; 10 for c3-f10)")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="c3", choices=sorted(workloads()))
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (reference kernel for the HBM byte counters)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step captured as HIP graphs (kernel figures from one eager step)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this implementation runs on one GPU only (the multi-GPU sharding is a design, "
              "not built); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
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
    kind = wl["kind"]
    stream = torch.cuda.current_stream()
    cfg = PL.StepConfig(B=B, beta=0.95, eps_rel=wl["eps_rel"], scale_mode=wl.get("scale", capi.SCALE_POWER),
                        solver=wl["solver"], variant=wl.get("variant", capi.NDB), iters=wl.get("iters", 10) or 10,
                        degree=wl.get("degree", 24), prec=wl["prec"], update_every=every)

    # Inputs, resident in HBM before anything is timed.
    tables = []
    if kind == "factors":
        A = W.config1_factors() if wl["cfg"] == 1 else W.config4_factors()
        cpu_inputs = A
        nf = A.shape[0]
        n = nf // 2
        Fd = torch.from_numpy(A).cuda()
        V0 = torch.from_numpy(W.start_vectors(wl["cfg"], nf, B)).cuda()
        scale, status = PL.new_scale(nf, "cuda")
        roots = torch.empty_like(Fd)
        wss = {"scale": PL.Workspace(), "root": PL.Workspace()}

        def do_scale():
            PL.scale_power(Fd, cfg.eps_rel, cfg.scale_mode, V0, cfg.pi_steps, cfg.safety, scale, status,
                           wss["scale"])

        def do_root():
            if cfg.solver == "newton":
                PL.invroot_newton(Fd, scale, cfg.p, cfg.variant, cfg.iters, roots, status, None, wss["root"])
            else:
                PL.invroot_cheby(Fd, scale, cfg.p, cfg.degree, cfg.interval_eps, cfg.prec, roots, status,
                                 wss["root"])

        def step(_t):
            do_scale()
            do_root()

        stage_fns = [("scale", do_scale), ("invroot", do_root)]
        status_of = lambda: status  # noqa: E731
    else:
        if kind == "stream":
            grads = [W.config2_gradient(t) for t in range(1, 6)]
            tens = [torch.from_numpy(g).cuda() for g in grads]
            outs = [torch.empty_like(t) for t in tens]
            tables = [(PL.BlockTable.from_layers([g], B), PL.BlockTable.from_layers([u], B))
                      for g, u in zip(tens, outs)]
            cpu_inputs = grads[:1]
        else:
            grads = W.model_gradients(wl["cfg"], wl["spec"])
            tens = [torch.from_numpy(g).cuda() for g in grads]
            outs = [torch.empty_like(t) for t in tens]
            k = wl["nblocks"]
            ge, ue = _entries(tens, B), _entries(outs, B)
            if k is not None:
                ge, ue = ge[:k], ue[:k]
            tables = [(PL.BlockTable(ge, B), PL.BlockTable(ue, B))]
            cpu_inputs = grads
        n = tables[0][0].n
        nf = 2 * n
        state = PL.ShampooBlocks(cfg, n)
        state.set_start_vectors(torch.from_numpy(W.start_vectors(wl["cfg"], nf, B)).cuda())

        def step(t):
            g, u = tables[t % len(tables)]
            state.step(g, u)

        def stage_acc():
            PL.accumulate(tables[0][0], state.factors, cfg.beta, 1 - cfg.beta, cfg.prec, state.ws["acc"])

        def stage_scale():
            PL.scale_power(state.factors, cfg.eps_rel, cfg.scale_mode, state.v0, cfg.pi_steps, cfg.safety,
                           state.scale, state.status, state.ws["scale"])

        def stage_root():
            if cfg.solver == "newton":
                PL.invroot_newton(state.factors, state.scale, cfg.p, cfg.variant, cfg.iters, state.roots,
                                  state.status, None, state.ws["root"])
            else:
                PL.invroot_cheby(state.factors, state.scale, cfg.p, cfg.degree, cfg.interval_eps, cfg.prec,
                                 state.roots, state.status, state.ws["root"])

        def stage_pre():
            PL.precondition(state.roots, tables[0][0], tables[0][1], cfg.prec, state.ws["pre"])

        stage_fns = [("accumulate", stage_acc), ("scale", stage_scale), ("invroot", stage_root),
                     ("precondition", stage_pre)]
        status_of = lambda: state.status  # noqa: E731

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()

    # Per-stage split (one untimed step with events between the stages).
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(stage_fns) + 1)]
    ev[0].record()
    for i, (_, fn) in enumerate(stage_fns):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    stages = {name: ev[i].elapsed_time(ev[i + 1]) for i, (name, _) in enumerate(stage_fns)}

    graft_ms = None
    if kind == "model":
        # Grafted parameter update (reported beside the step, not part of it).
        params = [t.clone() for t in tens]
        moms = [torch.zeros_like(t) for t in tens]
        vels = [torch.zeros_like(t) for t in tens]
        gtabs = [tables[0][0], tables[0][1]] + [PL.BlockTable(_entries(ts, B)[:n], B) for ts in (params, moms, vels)]
        PL.graft_update(*gtabs, 1e-3, 0.9, 0.95, 1e-8, 1)
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        PL.graft_update(*gtabs, 1e-3, 0.9, 0.95, 1e-8, 2)
        g1.record()
        torch.cuda.synchronize()
        graft_ms = g0.elapsed_time(g1)
        del params, moms, vels, gtabs

    # Timing hook on every hooked kernel family during eager steps.
    def run_hooked(nsteps):
        cap = 64 * nsteps + 64
        kev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * cap)]
        for e in kev:
            e.record(stream)  # materialise the underlying HIP events
        torch.cuda.synchronize()
        handles = (ctypes.c_void_p * (2 * cap))(*[e.cuda_event for e in kev])
        fams = (ctypes.c_int32 * cap)()
        capi.check(capi.shampoo_timing_hook(capi.TIME_ALL, ctypes.addressof(handles), ctypes.addressof(fams), cap),
                   "timing hook")
        if kind != "factors":
            state.t = 0  # the steps start with a root refresh
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(nsteps):
            step(t)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        recorded = capi.shampoo_timing_count()
        capi.shampoo_timing_hook(capi.TIME_OFF, None, None, 0)
        if recorded >= cap:
            print("bench.py: timing hook capacity reached; kernel figures cover the first launches only",
                  file=sys.stderr)
        per = {}
        for i in range(recorded):
            per.setdefault(int(fams[i]), []).append(kev[2 * i].elapsed_time(kev[2 * i + 1]))
        return per, t1 - t0

    if args.graph:
        if kind == "factors":
            g = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                do_scale()
                do_root()
            replays = [g.replay]
        else:
            replays = [state.capture(gt, ut).replay for gt, ut in tables]
        hooked_steps = 1
        per_fam, _ = run_hooked(hooked_steps)  # kernel figures from one eager step
        if kind != "factors":
            state.t = 0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(args.steps):
            replays[t % len(replays)]()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    else:
        hooked_steps = args.steps
        per_fam, elapsed = run_hooked(hooked_steps)

    traffic_rec = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            traffic_rec = json.load(f)
    kernels = []
    for fam, durs in sorted(per_fam.items()):
        name, flops, nbytes, peak_flops = family_info(fam, wl, B, nf, capi)
        avg = sum(durs) / len(durs)
        tflops = flops / (avg * 1e-3) / 1e12
        gbs = nbytes / (avg * 1e-3) / 1e9
        # bound: whichever roofline is lower at this kernel's arithmetic intensity
        hbm = flops / nbytes < peak_flops * 1e12 / (PEAK_HBM * 1e9)
        rec = traffic_rec.get(f"{args.workload}:{FAMILY_KEYS[fam]}")
        digest = source_digest(family_sources(fam, wl, capi))
        traffic = rec.get("bytes_per_launch") if rec and rec.get("source_digest") == digest else None
        kernels.append({"family": FAMILY_KEYS[fam], "kernel": name, "launches_timed": len(durs),
                        "avg_launch_ms": round(avg, 4), "total_ms": round(sum(durs), 3),
                        "bound": "hbm" if hbm else "mfma",
                        "achieved": round(gbs if hbm else tflops, 2), "peak": PEAK_HBM if hbm else peak_flops,
                        "unit": "GB/s" if hbm else "TFLOP/s",
                        "frac": round((gbs / PEAK_HBM) if hbm else (tflops / peak_flops), 4),
                        "traffic": traffic, "flops_per_launch": flops, "bytes_per_launch": nbytes,
                        "tflops": round(tflops, 2), "mfma_frac": round(tflops / peak_flops, 4),
                        "gbs": round(gbs, 1)})
    ms_step = 1e3 * elapsed / args.steps
    value = nf * refreshes / elapsed
    status = status_of().cpu()
    roofline = None
    if kernels:
        top = max(kernels, key=lambda k: k["total_ms"])
        roofline = {"bound": top["bound"], "achieved": top["achieved"], "peak": top["peak"], "unit": top["unit"],
                    "frac": top["frac"], "traffic": top["traffic"], "kernel": top["kernel"],
                    "launches_timed": top["launches_timed"], "avg_launch_ms": top["avg_launch_ms"],
                    "flops_per_launch": top["flops_per_launch"], "bytes_per_launch": top["bytes_per_launch"],
                    "share_of_step": round(top["total_ms"] / hooked_steps / ms_step, 4)}
    half = wl["prec"] == capi.BF16_IN or (cfg.solver == "newton" and (cfg.variant & 0xff) == capi.CN_F16)
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
        "dtype": ("bf16-in/f32" if wl["prec"] == capi.BF16_IN else "f16-in/f32" if half else "f32"),
        "data": ("synthetic N(0, 0.02^2) gradients of the workload's weight shapes, seeded" if kind != "factors"
                 else "synthetic SPD factors of the workload's recipe, seeded"),
        "config": dict({"workload": wl["name"], "B": B, "blocks": n, "factors": nf},
                       **({"update_every": every} if every > 1 else {}),
                       **({"hip_graph": True} if args.graph else {})),
        "roofline": roofline,
        "kernels": kernels,
        "stages_ms": {k: round(v, 3) for k, v in stages.items()},
        "stage_rates": stage_rates(wl, cfg, B, n, nf, stages, capi),
        "invroot_blocks_per_s": round(nf / (stages["invroot"] * 1e-3), 2),
        "status_nonzero_factors": int((status != 0).sum()),
    }
    if graft_ms is not None:
        out["graft_update_ms"] = round(graft_ms, 3)
    out["env"] = env_info()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, cpu_inputs, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
