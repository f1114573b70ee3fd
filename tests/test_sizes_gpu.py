"""Parity at the extremes of the supported sizes, through properties that hold
at any size.

For a diagonal factor F = diag(d) every iterate of every solver is diagonal,
so the result is the scalar recurrence of the oracle applied to each d_i
(the scalar maps are pinned against the matrix iterations in the oracle's
own tests) and every off-diagonal entry must stay exactly zero.  This runs
the full tile grid, the power-iteration panels and the 64-bit indexing at
B = 8192 and B = 16384 without a float64 B^3 reference.  Many tiny factors
exercise the other end (large grids of small items)."""
import math

import numpy as np
import pytest
import torch

from oracle import shampoo_oracle as O
from inverse_root_preconditioning_amd import capi
from inverse_root_preconditioning_amd import pipeline as PL
from inverse_root_preconditioning_amd import workloads as W

from gpu_helpers import TOL_F32, dev, gpu_roots, gpu_scale, host, oracle_root, oracle_scale, report

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    capi.load()


def diag_factors(key, nf, B):
    g = W.rng(W.TAG_EDGE, key)
    return [g.uniform(0.05, 1.0, B).astype(np.float32) for _ in range(nf)]


def make_diag_stack(ds, B):
    F = torch.zeros((len(ds), B, B), dtype=torch.float32, device="cuda")
    for i, d in enumerate(ds):
        F[i].diagonal().copy_(torch.from_numpy(d))
    return F


def check_diagonal(X, refs, name, **kw):
    err = 0.0
    for i, ref in enumerate(refs):
        x = X[i]
        dg = host(x.diagonal())
        off = torch.count_nonzero(x - torch.diag(x.diagonal())).item()
        assert off == 0, f"{off} nonzero off-diagonal entries"
        err = max(err, O.relative_frobenius(dg, ref))
    report(name, err=err, **kw)
    assert err <= TOL_F32, err


@pytest.mark.slow
@pytest.mark.parametrize("B,nf,method,arg", [(16384, 1, "ndb", 3), (8192, 2, "cn", 4), (8192, 1, "cheby", 8)])
def test_max_size_diagonal(B, nf, method, arg):
    ds = diag_factors(B + nf, nf, B)
    F = make_diag_stack(ds, B)
    V0 = W.start_vectors(77, nf, B)
    sc, st = gpu_scale(F, 1e-3, capi.SCALE_POWER, dev(V0), 20, 2.0)
    s = host(sc)
    refs = []
    for i, d in enumerate(ds):
        # oracle scale on the dense diagonal matrix (the same function as everywhere)
        o = O.scale_factor(np.diag(d.astype(np.float64)), 1e-3, "power", V0[i], 20, 2.0)
        assert abs(s[i, 0] - o["c"]) <= 1e-5 * o["c"] and abs(s[i, 1] - o["eps"]) <= 1e-5 * o["eps"]
        a = (d.astype(np.float64) + o["eps"]) / o["c"]
        if method == "ndb":
            phi = O.ndb_scalar(a, arg, "Y")
        elif method == "cn":
            phi = O.cn_scalar(a, 4, arg)
        else:
            phi = O.cheby_scalar(a, O.chebyshev_coefficients(arg, 4, 1e-12))
        refs.append(o["c"] ** -0.25 * phi)
    del V0
    if method == "ndb":
        X, _ = gpu_roots(F, sc, st, "newton", iters=arg, variant=capi.NDB)
    elif method == "cn":
        X, _ = gpu_roots(F, sc, st, "newton", iters=arg, variant=capi.CN)
    else:
        X, _ = gpu_roots(F, sc, st, "cheby", degree=arg)
    check_diagonal(X, refs, "max_size_diagonal", B=B, method=method)
    del X, F
    torch.cuda.empty_cache()


def test_max_size_accumulate_and_precondition_diagonal():
    """G = diag(g) at B = 16384: L = R = gamma diag(g^2) exactly, and with X = diag(x)
    the update is diag(x_L g x_R)."""
    B = 16384
    g = W.rng(W.TAG_EDGE, 91).uniform(-1.0, 1.0, B).astype(np.float32)
    G = torch.zeros((B, B), dtype=torch.float32, device="cuda")
    G.diagonal().copy_(torch.from_numpy(g))
    table = PL.BlockTable([(G, 0, 0, B, B)], B)
    F = torch.zeros((2, B, B), dtype=torch.float32, device="cuda")
    PL.accumulate(table, F, 0.0, 0.05)
    g64 = g.astype(np.float64)
    check_diagonal(F, [0.05 * g64 * g64, 0.05 * g64 * g64], "max_size_accumulate", B=B)
    del F
    xl = W.rng(W.TAG_EDGE, 92).uniform(0.5, 2.0, B).astype(np.float32)
    xr = W.rng(W.TAG_EDGE, 93).uniform(0.5, 2.0, B).astype(np.float32)
    X = make_diag_stack([xl, xr], B)
    U = torch.full_like(G, float("nan"))
    PL.precondition(X, table, PL.BlockTable([(U, 0, 0, B, B)], B))
    check_diagonal(U[None], [xl.astype(np.float64) * g64 * xr.astype(np.float64)], "max_size_precondition", B=B)


def test_many_small_factors():
    """4096 factors of 64 x 64 in one launch; sampled factors against the oracle."""
    nf, B = 4096, 64
    F = np.concatenate([W.spd_factors(200 + j, 512, B, cond=1e3) for j in range(nf // 512)])
    V0 = W.start_vectors(201, nf, B)
    Fd = dev(F)
    sc, st = gpu_scale(Fd, 1e-6, capi.SCALE_POWER, dev(V0))
    X, _ = gpu_roots(Fd, sc, st, "newton", iters=8, variant=capi.NDB)
    err = 0.0
    for i in (0, 1, 777, 2048, nf - 1):
        o = oracle_scale(F[i], 1e-6, capi.SCALE_POWER, V0[i])
        err = max(err, O.relative_frobenius(host(X[i]), oracle_root(F[i], o, "newton", iters=8)))
    report("many_small_factors", err=err)
    assert err <= TOL_F32
