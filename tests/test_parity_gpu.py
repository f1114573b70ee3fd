"""Stage-by-stage parity of the HIP path (through the C ABI) with the float64
oracle on seeded inputs, at sizes that span several tiles, plus the edge
cases of the method.  Tolerances: relative Frobenius per factor <= 1e-4 for
fp32 paths and <= 2e-2 for bf16-input paths."""
import math

import numpy as np
import pytest
import torch

from oracle import shampoo_oracle as O
from inverse_root_preconditioning_amd import capi
from inverse_root_preconditioning_amd import pipeline as PL
from inverse_root_preconditioning_amd import workloads as W

from gpu_helpers import (TOL_BF16, TOL_F32, dev, fill_factor, gpu_roots, gpu_scale, host, oracle_root,
                         oracle_scale, report, upper_tiles)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    capi.load()
    torch.manual_seed(0)


def grads(key, n, B, std=1.0):
    return np.stack([(W.rng(W.TAG_EDGE, key, i).standard_normal((B, B)) * std).astype(np.float32)
                     for i in range(n)])


# ---------------------------------------------------------------------------
# accumulate
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B,n", [(64, 3), (128, 3), (192, 3), (256, 3), (256, 86)])
def test_accumulate_gram_matches_oracle(B, n):
    """n = 86 blocks of 256 fill the GPU with 128 x 128 tiles (3 upper tiles
    each), the descriptor kernel the model-shaped steps run; fewer blocks run
    64 x 64 tiles.  The first three blocks are checked."""
    G = grads(1, n, B, 0.02)
    g = dev(G)
    table = PL.BlockTable.from_stack(g)
    F = torch.zeros((2 * n, B, B), dtype=torch.float32, device="cuda")
    PL.accumulate(table, F, 0.0, 1.0)
    out = host(F)
    for i in range(3):
        L, R = O.accumulate(np.zeros((B, B)), np.zeros((B, B)), G[i], 0.0, 1.0)
        el, er = O.relative_frobenius(out[i], L), O.relative_frobenius(out[n + i], R)
        assert el <= 1e-5 and er <= 1e-5, (el, er)
        assert np.array_equal(out[i], out[i].T) and np.array_equal(out[n + i], out[n + i].T)
    report("accumulate_gram", B=B, n=n, err=max(el, er))


def test_accumulate_ema_ragged_blocks():
    """Partial edge blocks (a 300 x 200 and a 128 x 70 gradient at B = 128),
    misaligned rows (ld = 70) and an EMA on top of an existing state."""
    B = 128
    A1 = W.ragged_gradients(2, [(300, 200)], 0.5)[0]
    A2 = W.ragged_gradients(3, [(128, 70)], 0.5)[0]
    t1, t2 = dev(A1), dev(A2)
    table = PL.BlockTable.from_layers([t1, t2], B)
    n = table.n
    assert n == 3 * 2 + 1
    prev = grads(4, 2 * n, B, 0.1)
    prevF = np.einsum("nij,nkj->nik", prev, prev).astype(np.float32)  # symmetric PSD start
    F = dev(prevF)
    PL.accumulate(table, F, 0.9, 0.1)
    out = host(F)
    blocks = []
    for t in (A1, A2):
        m, k = t.shape
        for r0 in range(0, m, B):
            for c0 in range(0, k, B):
                blocks.append(O.pad_block(t[r0:r0 + B, c0:c0 + B], B))
    err = 0.0
    for i, Gb in enumerate(blocks):
        L, R = O.accumulate(prevF[i], prevF[n + i], Gb, 0.9, 0.1)
        err = max(err, O.relative_frobenius(out[i], L), O.relative_frobenius(out[n + i], R))
    assert err <= 1e-5
    report("accumulate_ema_ragged", err=err)


def test_accumulate_bf16_input():
    B, n = 256, 4
    G = grads(5, n, B, 0.02)
    g = dev(G)
    F = torch.zeros((2 * n, B, B), dtype=torch.float32, device="cuda")
    PL.accumulate(PL.BlockTable.from_stack(g), F, 0.0, 1.0, prec=capi.BF16_IN)
    out = host(F)
    err = 0.0
    for i in range(n):
        L, R = O.accumulate(np.zeros((B, B)), np.zeros((B, B)), G[i], 0.0, 1.0)
        err = max(err, O.relative_frobenius(out[i], L), O.relative_frobenius(out[n + i], R))
    assert err <= TOL_BF16
    report("accumulate_bf16", err=err)


# ---------------------------------------------------------------------------
# scale
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B,r", [(64, 32), (192, 32), (256, 7), (768, 32), (1024, 20)])
def test_scale_power_matches_oracle(B, r):
    """B = 64 and 192 run the 64-row panel step, the others the 256-column
    panels read by columns after the first step (3 and 4 panels per factor)."""
    nf = 6
    F = W.spd_factors(10 + B, nf, B, cond=1e4) * np.float32(3.0)
    V0 = W.start_vectors(9, nf, B, r)
    sc, st = gpu_scale(dev(F), 1e-3, capi.SCALE_POWER, dev(V0), 20, 2.0)
    s, stt = host(sc), host(st)
    err = 0.0
    for i in range(nf):
        o = oracle_scale(F[i], 1e-3, capi.SCALE_POWER, V0[i])
        assert stt[i] == o["status"] == 0
        for k, key in enumerate(("c", "eps", "lam", "trace")):
            e = abs(s[i, k] - o[key]) / abs(o[key])
            err = max(err, e)
            assert e <= 2e-5, (key, s[i, k], o[key])
    report("scale_power", B=B, r=r, err=err)


@pytest.mark.parametrize("mode", [capi.SCALE_POWER, capi.SCALE_FROBENIUS])
@pytest.mark.parametrize("mag", [1e30, 1e-30])
def test_scale_and_roots_far_from_unit_magnitude(mode, mag):
    """Factors with eigenvalues up to 1e30 (or down to 1e-33): the squares the
    power iteration and the Frobenius norm form would leave fp32's range, so
    the scale stage works on F 2^-e with 2^e near the mean eigenvalue; c, the
    estimate and the roots still match the oracle, with no status bit."""
    nf, B = 4, 256
    F = (W.spd_factors(220, nf, B, cond=1e3).astype(np.float64) * mag).astype(np.float32)
    V0 = W.start_vectors(221, nf, B)
    Fd = dev(F)
    # eps_rel = 1e-6 keeps eps a normal fp32 number at both magnitudes
    sc, st = gpu_scale(Fd, 1e-6, mode, dev(V0), 20, 2.0)
    X, _ = gpu_roots(Fd, sc, st, "newton", iters=6, p=4, variant=capi.NDB_Z)
    s, stt, Xh = host(sc), host(st), host(X)
    err = 0.0
    for i in range(nf):
        o = oracle_scale(F[i], 1e-6, mode, V0[i])
        assert stt[i] == o["status"] == 0, (i, stt[i])
        for k, key in enumerate(("c", "eps", "lam", "trace")):
            e = abs(s[i, k] - o[key]) / abs(o[key])
            assert e <= 2e-5, (key, s[i, k], o[key])
        err = max(err, O.relative_frobenius(Xh[i], oracle_root(F[i], o, "newton", iters=6, variant=capi.NDB_Z)))
    assert err <= TOL_F32, err
    report("scale_range", mode=mode, mag=mag, root_err=err)


def test_scale_frobenius_matches_oracle():
    nf, B = 5, 128
    F = W.spd_factors(20, nf, B, cond=1e2)
    sc, st = gpu_scale(dev(F), 1e-2, capi.SCALE_FROBENIUS)
    s = host(sc)
    for i in range(nf):
        o = oracle_scale(F[i], 1e-2, capi.SCALE_FROBENIUS, None)
        assert abs(s[i, 0] - o["c"]) / o["c"] <= 1e-5
        assert abs(s[i, 3] - o["trace"]) / o["trace"] <= 1e-5


# ---------------------------------------------------------------------------
# inverse roots
# ---------------------------------------------------------------------------

NEWTON_CASES = [
    (capi.NDB, 4, 1), (capi.NDB, 4, 2), (capi.NDB, 4, 6), (capi.NDB_Z, 4, 1), (capi.NDB_Z, 4, 6),
    (capi.NDB, 2, 5), (capi.CN, 4, 1), (capi.CN, 4, 2), (capi.CN, 4, 8), (capi.CN, 1, 6), (capi.CN, 2, 6),
    (capi.CN, 8, 6),
]


@pytest.mark.parametrize("full", [False, True])
@pytest.mark.parametrize("B", [64, 256])
@pytest.mark.parametrize("variant,p,iters", NEWTON_CASES)
def test_newton_matches_oracle(B, variant, p, iters, full):
    nf = 4
    F = W.spd_factors(30 + B, nf, B, cond=1e3)
    V0 = W.start_vectors(31, nf, B)
    Fd = dev(F)
    sc, st = gpu_scale(Fd, 0.0, capi.SCALE_POWER, dev(V0))
    v = variant | (capi.FULL_PRODUCTS if full else 0)
    X, R = gpu_roots(Fd, sc, st, "newton", iters=iters, p=p, variant=v, resid=True)
    Xh, Rh = host(X), host(R)
    err = 0.0
    for i in range(nf):
        o = oracle_scale(F[i], 0.0, capi.SCALE_POWER, V0[i])
        ref = oracle_root(F[i], o, "newton", iters=iters, p=p, variant=variant)
        err = max(err, O.relative_frobenius(Xh[i], ref))
    assert err <= TOL_F32, err
    assert np.all(Rh >= 0.0) and np.all(np.isfinite(Rh))
    if not full and not (variant == capi.CN and iters > 1):
        # products of commuting polynomials are formed from upper tiles: exactly symmetric
        assert all(np.array_equal(Xh[i], Xh[i].T) for i in range(nf))
    report("newton", B=B, variant=variant, p=p, iters=iters, full=full, err=err)


SPAN_CASES = [("newton", capi.NDB_Z, 6, False), ("newton", capi.NDB, 6, False), ("newton", capi.NDB_Z, 6, True),
              ("newton", capi.CN, 6, False), ("cheby", None, 16, False)]


@pytest.mark.parametrize("B,solver,variant,arg,full",
                         [(B,) + c for B in (512, 640, 768) for c in SPAN_CASES] +
                         [(1280,) + SPAN_CASES[0], (1280,) + SPAN_CASES[3], (1280,) + SPAN_CASES[4]])
def test_fp32_products_span_tiles(B, solver, variant, arg, full):
    """fp32 roots on several output tiles per factor: B = 512 runs the 256 x 256
    direct-to-LDS kernel on 2 x 2 tiles (3 upper tiles, two of them diagonal),
    B = 768 on 3 x 3 and B = 1280 on 5 x 5 (15 upper tiles; the coupled-Newton
    C^p M product with its epilogue through LDS), B = 640 the 128 x 128 kernel
    on 5 x 5 tiles; symmetric and full products, reductions and epilogues all
    cross tile boundaries.  The three checked factors are replicated until a
    symmetric product's grid fills the GPU (below that the library picks
    smaller tiles); every copy must give the same bits."""
    base = 3
    T = 256 if B % 256 == 0 else 128
    reps = fill_factor(B, upper_tiles(B, T), base)
    nf = base * reps
    F = np.concatenate([W.spd_factors(70 + B, base, B, cond=1e3)] * reps)
    V0 = np.concatenate([W.start_vectors(71, base, B)] * reps)
    Fd = dev(F)
    sc, st = gpu_scale(Fd, 0.0, capi.SCALE_POWER, dev(V0))
    if solver == "newton":
        v = variant | (capi.FULL_PRODUCTS if full else 0)
        X, R = gpu_roots(Fd, sc, st, "newton", iters=arg, p=4, variant=v, resid=True)
        assert np.all(np.isfinite(host(R)))
    else:
        X, _ = gpu_roots(Fd, sc, st, "cheby", degree=arg, prec=capi.F32)
    Xh = host(X)
    assert all(np.array_equal(Xh[i], Xh[i % base]) for i in range(nf))
    err = 0.0
    for i in range(base):
        o = oracle_scale(F[i], 0.0, capi.SCALE_POWER, V0[i])
        if solver == "newton":
            ref = oracle_root(F[i], o, "newton", iters=arg, p=4, variant=variant)
        else:
            ref = oracle_root(F[i], o, "cheby", degree=arg)
        err = max(err, O.relative_frobenius(Xh[i], ref))
    assert err <= TOL_F32, err
    if not full and variant != capi.CN:
        assert all(np.array_equal(Xh[i], Xh[i].T) for i in range(base))
    report("fp32_span_tiles", B=B, solver=solver, variant=variant, arg=arg, full=full, nf=nf, err=err)


def test_newton_db_residuals_match_oracle():
    nf, B, k = 3, 128, 5
    F = W.spd_factors(40, nf, B, cond=1e2)
    V0 = W.start_vectors(41, nf, B)
    Fd = dev(F)
    sc, st = gpu_scale(Fd, 0.0, capi.SCALE_POWER, dev(V0))
    _, R = gpu_roots(Fd, sc, st, "newton", iters=k, p=4, variant=capi.NDB, resid=True)
    Rh = host(R)
    for i in range(nf):
        o = oracle_scale(F[i], 0.0, capi.SCALE_POWER, V0[i])
        A_s = O.damped(F[i], o["eps"]) / o["c"]
        _, res = O.invroot_newton_db(A_s, k, "Y")
        assert np.allclose(Rh[i], res, rtol=1e-3, atol=1e-5), (Rh[i], res)


_RESID_CACHE = {}


def _oracle_residuals(B, variant, iters):
    """(F, V0, per-factor oracle residual lists) for the large-kernel residual tests."""
    key = (B, variant, iters)
    if key not in _RESID_CACHE:
        nf = 2
        F = W.spd_factors(200 + B, nf, B, cond=1e3)
        V0 = W.start_vectors(201, nf, B)
        refs = []
        for i in range(nf):
            o = oracle_scale(F[i], 0.0, capi.SCALE_POWER, V0[i])
            A_s = O.damped(F[i], o["eps"]) / o["c"]
            if variant in (capi.CN, capi.CN_F16):
                refs.append(O.coupled_newton(A_s, 4, iters)[1])
            else:
                refs.append(O.invroot_newton_db(A_s, iters, "Z" if variant == capi.NDB_Z else "Y")[1])
        _RESID_CACHE[key] = (F, V0, np.array(refs))
    return _RESID_CACHE[key]


@pytest.mark.parametrize("mode", ["sym", "full", "sym_coupling"])
@pytest.mark.parametrize("variant", [capi.NDB, capi.NDB_Z, capi.CN])
@pytest.mark.parametrize("B", [512, 1024])
def test_residuals_match_oracle_large_kernel(B, variant, mode):
    """The per-iteration residuals (||I - Z Y||_F of both Newton-DB passes,
    ||I - M||_F of coupled Newton) that the 256 x 256 fp32 kernel's epilogue
    reduces, against the float64 iteration's: with the coupling product in
    full (default), every product in full, and the coupling product from upper
    tiles (diagonal tiles' upper entries weighted twice).  Above the fp32
    rounding floor the residuals agree to 1e-3 relative; at the floor (about
    1e-4 here) the computed value measures rounding, and is bounded by 1e-3."""
    iters = 6
    F, V0, ref = _oracle_residuals(B, variant, iters)
    reps = fill_factor(B, upper_tiles(B, 256), F.shape[0])  # the 256 x 256 kernel, as the model-shaped steps
    Fd = dev(np.concatenate([F] * reps))
    sc, st = gpu_scale(Fd, 0.0, capi.SCALE_POWER, dev(np.concatenate([V0] * reps)))
    bits = {"sym": 0, "full": capi.FULL_PRODUCTS, "sym_coupling": capi.SYM_COUPLING}[mode]
    _, R = gpu_roots(Fd, sc, st, "newton", iters=iters, p=4, variant=variant | bits, resid=True)
    Rh, sth = host(R), host(st)
    assert all(np.array_equal(Rh[i], Rh[i % F.shape[0]]) for i in range(Rh.shape[0]))
    Rh = Rh[:F.shape[0]]
    assert Rh.shape == ref.shape
    live = ref > 1e-2
    rel = np.abs(Rh - ref) / np.where(live, ref, 1.0)
    assert np.all(rel[live] <= 1e-3), (Rh, ref)
    assert np.all(np.abs(Rh - ref)[~live] <= 1e-3), (Rh, ref)
    assert np.all(sth == 0)
    report("resid_large_kernel", B=B, variant=variant, mode=mode, max_rel=float(rel[live].max()),
           floor_max=float(np.abs(Rh - ref)[~live].max()) if (~live).any() else 0.0)


@pytest.mark.parametrize("B", [512, 1024])
def test_residuals_match_oracle_fp16_coupled_newton(B):
    """||I - M||_F from the epilogue of the fp16-operand C^p M product against
    the float64 coupled Newton: within the half-width bar, 2e-2 relative, while
    above fp16's rounding floor (bounded by 0.5 there)."""
    iters = 6
    F, V0, ref = _oracle_residuals(B, capi.CN_F16, iters)
    Fd = dev(F)
    sc, st = gpu_scale(Fd, 0.0, capi.SCALE_POWER, dev(V0))
    _, R = gpu_roots(Fd, sc, st, "newton", iters=iters, p=4, variant=capi.CN_F16, resid=True)
    Rh = host(R)
    live = ref > 1.0
    rel = np.abs(Rh - ref) / np.where(live, ref, 1.0)
    assert np.all(rel[live] <= TOL_BF16), (Rh, ref)
    assert np.all(np.abs(Rh - ref)[~live] <= 0.5), (Rh, ref)
    report("resid_cn_fp16", B=B, max_rel=float(rel[live].max()))


def test_binding_rejects_short_residual_and_status_tensors():
    nf, B = 2, 64
    F = dev(W.spd_factors(210, nf, B, cond=10.0))
    sc, st = PL.new_scale(nf, "cuda")
    X = torch.empty_like(F)
    short = torch.zeros((nf, 5), dtype=torch.float32, device="cuda")  # one pass of 5; Newton-DB p = 4 needs 10
    with pytest.raises(ValueError, match="resid_out"):
        PL.invroot_newton(F, sc, 4, capi.NDB, 5, X, st, short)
    with pytest.raises(ValueError, match="status"):
        PL.invroot_newton(F, sc, 4, capi.NDB, 5, X, st.to(torch.int64))
    with pytest.raises(ValueError, match="scale"):
        PL.invroot_cheby(F, sc[:1], 4, 8, 0.0, capi.F32, X, st)


@pytest.mark.parametrize("full", [False, True])
@pytest.mark.parametrize("B", [64, 128])
@pytest.mark.parametrize("degree", [1, 2, 3, 16, 32])
def test_chebyshev_f32_matches_oracle(B, degree, full):
    nf = 4
    F = W.spd_factors(50 + B, nf, B, cond=1e4)
    V0 = W.start_vectors(51, nf, B)
    Fd = dev(F)
    sc, st = gpu_scale(Fd, 0.0, capi.SCALE_POWER, dev(V0))
    X, _ = gpu_roots(Fd, sc, st, "cheby", degree=degree, prec=capi.F32 | (capi.FULL_PRODUCTS if full else 0))
    Xh = host(X)
    err = 0.0
    for i in range(nf):
        o = oracle_scale(F[i], 0.0, capi.SCALE_POWER, V0[i])
        err = max(err, O.relative_frobenius(Xh[i], oracle_root(F[i], o, "cheby", degree=degree)))
    assert err <= TOL_F32, err
    if not full:
        assert all(np.array_equal(Xh[i], Xh[i].T) for i in range(nf))
    report("cheby_f32", B=B, degree=degree, full=full, err=err)


@pytest.mark.parametrize("full", [False, True])
@pytest.mark.parametrize("degree", [2, 16, 24])
def test_chebyshev_bf16_matches_oracle(degree, full):
    nf, B = 4, 256
    F = W.spd_factors(60, nf, B, cond=1e4)
    V0 = W.start_vectors(61, nf, B)
    Fd = dev(F)
    sc, st = gpu_scale(Fd, 0.0, capi.SCALE_POWER, dev(V0))
    X, _ = gpu_roots(Fd, sc, st, "cheby", degree=degree,
                     prec=capi.BF16_IN | (capi.FULL_PRODUCTS if full else 0))
    Xh = host(X)
    err = 0.0
    for i in range(nf):
        o = oracle_scale(F[i], 0.0, capi.SCALE_POWER, V0[i])
        err = max(err, O.relative_frobenius(Xh[i], oracle_root(F[i], o, "cheby", degree=degree)))
    assert err <= TOL_BF16, err
    report("cheby_bf16", degree=degree, full=full, err=err)


# ---------------------------------------------------------------------------
# precondition
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("prec,tol", [(capi.F32, 1e-5), (capi.BF16_IN, TOL_BF16)])
def test_precondition_ragged(prec, tol):
    B = 128
    A1 = W.ragged_gradients(7, [(260, 300)], 1.0)[0]
    t1 = dev(A1)
    gt = PL.BlockTable.from_layers([t1], B)
    n = gt.n
    X = np.concatenate([W.spd_factors(70, n, B, cond=10.0), W.spd_factors(71, n, B, cond=10.0)])
    U = torch.full_like(t1, float("nan"))
    ut = PL.BlockTable.from_layers([U], B)
    PL.precondition(dev(X), gt, ut, prec=prec)
    Uh = host(U)
    assert np.all(np.isfinite(Uh)), "some part of U was not written"
    err = 0.0
    i = 0
    for r0 in range(0, A1.shape[0], B):
        for c0 in range(0, A1.shape[1], B):
            g = O.pad_block(A1[r0:r0 + B, c0:c0 + B], B)
            ref = O.precondition(X[i], g, X[n + i])
            rows, cols = min(B, A1.shape[0] - r0), min(B, A1.shape[1] - c0)
            err = max(err, O.relative_frobenius(Uh[r0:r0 + rows, c0:c0 + cols], ref[:rows, :cols]))
            i += 1
    assert err <= tol, err
    report("precondition", prec=prec, err=err)


# ---------------------------------------------------------------------------
# degenerate factors, empty input, determinism
# ---------------------------------------------------------------------------

def test_degenerate_factors():
    B = 64
    good = W.spd_factors(80, 1, B, cond=10.0)[0]
    zero = np.zeros((B, B), np.float32)
    neg = -good
    bad = good.copy()
    bad[3, 5] = np.nan
    F = np.stack([good, zero, neg, bad])
    V0 = W.start_vectors(81, 4, B)
    Fd = dev(F)
    sc, st = gpu_scale(Fd, 1e-12, capi.SCALE_POWER, dev(V0))
    s = host(st)
    for i in range(4):
        assert s[i] == oracle_scale(F[i], 1e-12, capi.SCALE_POWER, V0[i])["status"], (i, s)
    assert s[0] == 0 and s[1] == capi.BLK_ZERO and s[2] == capi.BLK_NONPOS_RQ and s[3] & capi.BLK_NONFINITE
    for method in ("newton", "cheby"):
        X, _ = gpu_roots(Fd, sc, st, method, iters=4, degree=8)
        Xh = host(X)
        assert np.array_equal(Xh[1], np.eye(B)) and np.array_equal(Xh[2], np.eye(B))
        assert np.all(np.isfinite(Xh[0])) and not np.all(np.isfinite(Xh[3]))
    s2 = host(st)
    assert s2[3] & capi.BLK_NONFINITE


def test_empty_input_is_noop():
    F = torch.zeros((0, 64, 64), dtype=torch.float32, device="cuda")
    sc, st = PL.new_scale(0, "cuda")
    ws = PL.Workspace()
    p, nb = ws.get(256)
    assert capi.shampoo_invroot_newton(F.data_ptr(), sc.data_ptr(), 0, 64, 4, capi.NDB, 3, F.data_ptr(), 0,
                                       st.data_ptr(), p, nb, 0) == capi.OK


def test_repeat_runs_are_bitwise_identical():
    nf, B = 6, 256
    F = W.spd_factors(90, nf, B, cond=1e5)
    V0 = W.start_vectors(91, nf, B)
    Fd, Vd = dev(F), dev(V0)
    outs = []
    for _ in range(2):
        sc, st = gpu_scale(Fd, 1e-12, capi.SCALE_POWER, Vd)
        X, R = gpu_roots(Fd, sc, st, "newton", iters=7, variant=capi.NDB, resid=True)
        outs.append((host(sc), host(X), host(R)))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)


def test_repeat_runs_are_bitwise_identical_large_tiles():
    """The same on 2 x 2 large tiles: power iteration by columns, Newton-DB on
    the fp32 large kernel and bf16 Chebyshev on the 8-wave 16-bit kernel with
    their LDS-staged symmetric epilogues (fixed reduction orders throughout)."""
    B = 512
    reps = fill_factor(B, upper_tiles(B, 256), 3)
    F = np.concatenate([W.spd_factors(92, 3, B, cond=1e4)] * reps)
    V0 = np.concatenate([W.start_vectors(93, 3, B)] * reps)
    Fd, Vd = dev(F), dev(V0)
    outs = []
    for _ in range(2):
        sc, st = gpu_scale(Fd, 1e-12, capi.SCALE_POWER, Vd)
        X, R = gpu_roots(Fd, sc, st, "newton", iters=5, variant=capi.NDB_Z, resid=True)
        Xc, _ = gpu_roots(Fd, sc, st, "cheby", degree=12, prec=capi.BF16_IN)
        outs.append((host(sc), host(X), host(R), host(Xc)))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("full", [False, True])
@pytest.mark.parametrize("B", [128, 256])
@pytest.mark.parametrize("p,iters", [(4, 1), (4, 2), (4, 6), (4, 12), (1, 6), (2, 6), (8, 6)])
def test_coupled_newton_fp16_matches_oracle(B, p, iters, full):
    """Coupled Newton on fp16 operands with fp32 accumulation, against the
    float64 coupled Newton (half-width-input tolerance 2e-2)."""
    nf = 4
    F = W.spd_factors(130 + B, nf, B, cond=1e3)
    V0 = W.start_vectors(131, nf, B)
    Fd = dev(F)
    sc, st = gpu_scale(Fd, 0.0, capi.SCALE_POWER, dev(V0))
    v = capi.CN_F16 | (capi.FULL_PRODUCTS if full else 0)
    X, R = gpu_roots(Fd, sc, st, "newton", iters=iters, p=p, variant=v, resid=True)
    Xh, Rh = host(X), host(R)
    err = 0.0
    for i in range(nf):
        o = oracle_scale(F[i], 0.0, capi.SCALE_POWER, V0[i])
        err = max(err, O.relative_frobenius(Xh[i], oracle_root(F[i], o, "newton", iters=iters, p=p,
                                                                variant=capi.CN)))
    assert err <= TOL_BF16, err
    assert np.all(np.isfinite(Rh)) and np.all(Rh >= 0.0)
    report("cn_fp16", B=B, p=p, iters=iters, full=full, err=err)


@pytest.mark.parametrize("sym_c", [False, True])
@pytest.mark.parametrize("B", [512, 768])
@pytest.mark.parametrize("p,iters", [(1, 5), (2, 5), (4, 5), (8, 4)])
def test_coupled_newton_fp16_upper_operands(B, p, iters, sym_c):
    """With B a multiple of 256, fp16 coupled Newton keeps the fp16 results of
    its symmetric products (X C, C^2, C^4, ...) on and above the diagonal only,
    and the next products read the lower tiles of their panels transposed from
    there: as the left operand (X C, C^p M, the final X C), as both operands
    (C^2 C^2), in symmetric and full C^p M products.  2 x 2 and 3 x 3 tiles
    per factor, each p, against the float64 coupled Newton."""
    nf = 2
    F = W.spd_factors(170 + B + p, nf, B, cond=1e3)
    V0 = W.start_vectors(171, nf, B)
    Fd = dev(F)
    sc, st = gpu_scale(Fd, 0.0, capi.SCALE_POWER, dev(V0))
    v = capi.CN_F16 | (capi.SYM_COUPLING if sym_c else 0)
    X, R = gpu_roots(Fd, sc, st, "newton", iters=iters, p=p, variant=v, resid=True)
    Xh, Rh = host(X), host(R)
    err = 0.0
    for i in range(nf):
        o = oracle_scale(F[i], 0.0, capi.SCALE_POWER, V0[i])
        err = max(err, O.relative_frobenius(Xh[i], oracle_root(F[i], o, "newton", iters=iters, p=p,
                                                                variant=capi.CN)))
        assert np.array_equal(Xh[i], Xh[i].T)
    assert err <= TOL_BF16, err
    assert np.all(np.isfinite(Rh)) and np.all(Rh >= 0.0)
    report("cn_fp16_upper", B=B, p=p, iters=iters, sym_c=sym_c, err=err)


@pytest.mark.parametrize("B", [384, 512, 1280])
def test_accumulate_bf16_ema_over_prior_state(B):
    """bf16-input EMA steps over a nonzero state, two in a row, each checked
    against the oracle's step from the GPU's previous state: the old factor
    enters through the epilogue's loads (on the 256 x 256 tiles requested
    groups ahead, at each entry's own position, with the factor updated in
    place).  The prior is a Gram matrix of the product's own size with weight
    0.9, so an entry read from the wrong place would be an O(1) error; the
    state must stay exactly symmetric."""
    n = 2
    G0, G1, G2 = (grads(170 + B + t, n, B, 0.02) for t in range(3))
    prior = np.stack([m for i in range(n) for m in O.accumulate(np.zeros((B, B)), np.zeros((B, B)), G0[i], 0.0, 1.0)])
    prior = np.concatenate([prior[0::2], prior[1::2]]).astype(np.float32)  # all L, then all R
    F = dev(prior)
    for t, G in enumerate((G1, G2)):
        prev = host(F).astype(np.float64)
        PL.accumulate(PL.BlockTable.from_stack(dev(G)), F, 0.9, 0.1, prec=capi.BF16_IN)
        out = host(F)
        err = 0.0
        for i in range(n):
            L, R = O.accumulate(prev[i], prev[n + i], G[i], 0.9, 0.1)
            err = max(err, O.relative_frobenius(out[i], L), O.relative_frobenius(out[n + i], R))
            assert np.array_equal(out[i], out[i].T) and np.array_equal(out[n + i], out[n + i].T)
        assert err <= TOL_BF16, (t, err)
        report("accumulate_bf16_ema", B=B, step=t, err=err)


@pytest.mark.parametrize("B", [384, 512, 1280])
def test_half_width_products_span_tiles(B):
    """The 16-bit products on several tiles per factor: B = 384 runs the
    128 x 128 workgroup tile (3 x 3 tiles), B = 512 and 1280 the 256 x 256 ones
    (2 x 2 and 5 x 5),
    both with off-diagonal symmetric tiles and their mirrored writes:
    bf16-input accumulation, Chebyshev (symmetric and full products), coupled
    Newton on fp16 operands (with its tile reductions) and preconditioning."""
    nf, n = 2, 2
    G = grads(150 + B, n, B, 0.02)
    F = torch.zeros((2 * n, B, B), dtype=torch.float32, device="cuda")
    PL.accumulate(PL.BlockTable.from_stack(dev(G)), F, 0.0, 1.0, prec=capi.BF16_IN)
    out = host(F)
    err = 0.0
    for i in range(n):
        L, R = O.accumulate(np.zeros((B, B)), np.zeros((B, B)), G[i], 0.0, 1.0)
        err = max(err, O.relative_frobenius(out[i], L), O.relative_frobenius(out[n + i], R))
        assert np.array_equal(out[i], out[i].T) and np.array_equal(out[n + i], out[n + i].T)
    assert err <= TOL_BF16, err
    report("h16_tiles_accumulate", B=B, err=err)

    Fs = W.spd_factors(151 + B, nf, B, cond=1e3)
    V0 = W.start_vectors(152, nf, B)
    Fd = dev(Fs)
    sc, st = gpu_scale(Fd, 0.0, capi.SCALE_POWER, dev(V0))
    os_ = [oracle_scale(Fs[i], 0.0, capi.SCALE_POWER, V0[i]) for i in range(nf)]
    for full in (False, True):
        X, _ = gpu_roots(Fd, sc, st, "cheby", degree=8, prec=capi.BF16_IN | (capi.FULL_PRODUCTS if full else 0))
        Xh = host(X)
        err = max(O.relative_frobenius(Xh[i], oracle_root(Fs[i], os_[i], "cheby", degree=8)) for i in range(nf))
        assert err <= TOL_BF16, err
        if not full:
            assert all(np.array_equal(Xh[i], Xh[i].T) for i in range(nf))
        report("h16_tiles_cheby", B=B, full=full, err=err)
    X, R = gpu_roots(Fd, sc, st, "newton", iters=4, p=4, variant=capi.CN_F16, resid=True)
    Xh, Rh = host(X), host(R)
    err = max(O.relative_frobenius(Xh[i], oracle_root(Fs[i], os_[i], "newton", iters=4, p=4, variant=capi.CN))
              for i in range(nf))
    assert err <= TOL_BF16, err
    assert np.all(np.isfinite(Rh)) and np.all(Rh >= 0.0)
    report("h16_tiles_cn_fp16", B=B, err=err)

    Xp = np.concatenate([W.spd_factors(153 + B, n, B, cond=10.0), W.spd_factors(154 + B, n, B, cond=10.0)])
    U = torch.full((n, B, B), float("nan"), dtype=torch.float32, device="cuda")
    PL.precondition(dev(Xp), PL.BlockTable.from_stack(dev(G)), PL.BlockTable.from_stack(U), prec=capi.BF16_IN)
    Uh = host(U)
    err = max(O.relative_frobenius(Uh[i], O.precondition(Xp[i], G[i], Xp[n + i])) for i in range(n))
    assert err <= TOL_BF16, err
    report("h16_tiles_precondition", B=B, err=err)


@pytest.mark.parametrize("B,variant,iters,tol", [(256, capi.NDB_Z, 6, TOL_F32), (256, capi.NDB, 6, TOL_F32),
                                                (256, capi.CN, 8, TOL_F32), (256, capi.CN_F16, 8, TOL_BF16),
                                                (768, capi.NDB_Z, 6, TOL_F32), (768, capi.CN, 6, TOL_F32)])
def test_symmetric_coupling_opt_in(B, variant, iters, tol):
    """SHAMPOO_SYM_COUPLING forms Z Y (and C^p M) from upper tiles: on moderately
    conditioned factors and a few iterations it matches the oracle like the
    default, its residuals agree with the default's, and the roots are exactly
    symmetric.  B = 768 runs Z Y on 3 x 3 tiles of the large kernel (three
    diagonal tiles, reductions standing for mirrored tiles)."""
    nf = 4
    reps = fill_factor(B, upper_tiles(B, 256), nf) if B >= 512 else 1
    F = np.concatenate([W.spd_factors(160, nf, B, cond=1e3)] * reps)
    V0 = np.concatenate([W.start_vectors(161, nf, B)] * reps)
    Fd = dev(F)
    sc, st = gpu_scale(Fd, 0.0, capi.SCALE_POWER, dev(V0))
    X, R = gpu_roots(Fd, sc, st, "newton", iters=iters, p=4, variant=variant | capi.SYM_COUPLING, resid=True)
    _, R0 = gpu_roots(Fd, sc, st, "newton", iters=iters, p=4, variant=variant, resid=True)
    Xh, Rh, R0h = host(X)[:nf], host(R)[:nf], host(R0)[:nf]
    base = capi.CN if variant == capi.CN_F16 else variant
    err = 0.0
    for i in range(nf):
        o = oracle_scale(F[i], 0.0, capi.SCALE_POWER, V0[i])
        err = max(err, O.relative_frobenius(Xh[i], oracle_root(F[i], o, "newton", iters=iters, p=4, variant=base)))
        assert np.array_equal(Xh[i], Xh[i].T)
    assert err <= tol, err
    # the weighted tile reductions give the same residual norms as the full products
    assert np.allclose(Rh, R0h, rtol=2e-2 if variant == capi.CN_F16 else 1e-3, atol=1e-4), (Rh, R0h)
    report("sym_coupling", B=B, variant=variant, iters=iters, err=err)
