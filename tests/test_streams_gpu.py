"""Streams: calls on different streams with distinct workspaces may run at
the same time.  Two factor sets go through scale, Newton-DB, the bf16
Chebyshev root and fp16 coupled Newton on two side streams at once (each
with its own workspace), and two whole optimizer states take two steps each
on two side streams at once; every result must equal, bit for bit, the same
calls run one after the other on the default stream (fixed reduction orders,
no shared state)."""
import numpy as np
import pytest
import torch

from inverse_root_preconditioning_amd import capi
from inverse_root_preconditioning_amd import pipeline as PL
from inverse_root_preconditioning_amd import workloads as W

from gpu_helpers import dev, fill_factor, host, upper_tiles

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    capi.load()


def _chain(F, V, ws, stream):
    nf = F.shape[0]
    sc, st = PL.new_scale(nf, F.device)
    PL.scale_power(F, 1e-12, capi.SCALE_POWER, V, 20, 2.0, sc, st, ws=ws, stream=stream)
    X = torch.empty_like(F)
    R = torch.empty((nf, 2 * 6), dtype=torch.float32, device=F.device)
    PL.invroot_newton(F, sc, 4, capi.NDB_Z, 6, X, st, R, ws=ws, stream=stream)
    Xc = torch.empty_like(F)
    PL.invroot_cheby(F, sc, 4, 12, 1e-12, capi.BF16_IN, Xc, st, ws=ws, stream=stream)
    Xh = torch.empty_like(F)
    PL.invroot_newton(F, sc, 4, capi.CN_F16, 6, Xh, st, ws=ws, stream=stream)
    return sc, st, X, R, Xc, Xh


def test_concurrent_streams_match_sequential():
    B = 512
    reps = fill_factor(B, upper_tiles(B, 256), 3)  # large-tile kernels, as the model-shaped steps run
    sets = []
    for key in (310, 320):
        F = np.concatenate([W.spd_factors(key, 3, B, cond=1e4)] * reps)
        V = np.concatenate([W.start_vectors(key + 1, 3, B)] * reps)
        sets.append((dev(F), dev(V)))
    torch.cuda.synchronize()
    ref = [[host(t) for t in _chain(F, V, PL.Workspace(), None)] for F, V in sets]

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    wss = [PL.Workspace(), PL.Workspace()]
    torch.cuda.synchronize()
    outs = []
    for (F, V), s, ws in zip(sets, streams, wss):
        with torch.cuda.stream(s):
            outs.append(_chain(F, V, ws, s))
    torch.cuda.synchronize()
    for r, o in zip(ref, outs):
        for a, b in zip(r, o):
            assert np.array_equal(a, host(b))


def _steps(cfg, grads, v0, stream):
    """Two optimizer steps (accumulate, scale, roots, precondition) of one state."""
    n = grads[0].shape[0]
    state = PL.ShampooBlocks(cfg, n)
    state.set_start_vectors(v0)
    outs = []
    for g in grads:
        u = torch.zeros_like(g)
        state.step(PL.BlockTable.from_stack(g), PL.BlockTable.from_stack(u), stream)
        outs.append(u)
    return [state.factors, state.roots, state.scale, state.status] + outs


def test_concurrent_optimizer_steps_match_sequential():
    B, n = 256, 24
    cfgs = [PL.StepConfig(B, variant=capi.NDB_Z, iters=8),
            PL.StepConfig(B, solver="cheby", degree=16, prec=capi.BF16_IN)]
    runs = []
    for k, cfg in enumerate(cfgs):
        grads = [dev(np.stack([W.gaussian((40 + k, 1, t, i), (B, B)) for i in range(n)])) for t in range(2)]
        v0 = dev(W.start_vectors(50 + k, 2 * n, B))
        runs.append((cfg, grads, v0))
    torch.cuda.synchronize()
    ref = [[host(t) for t in _steps(cfg, grads, v0, None)] for cfg, grads, v0 in runs]

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    torch.cuda.synchronize()
    outs = []
    for (cfg, grads, v0), s in zip(runs, streams):
        with torch.cuda.stream(s):
            outs.append(_steps(cfg, grads, v0, s))
    torch.cuda.synchronize()
    for r, o in zip(ref, outs):
        for a, b in zip(r, o):
            assert np.array_equal(a, host(b))
