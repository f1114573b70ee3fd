"""Why the coupling product P = Z Y of Newton-DB is computed in full by
default (SHAMPOO_SYM_COUPLING forms it from upper tiles, mirrored).

A small float32 emulation of the two forms on the CPU (numpy `@` for the
products; the symmetric form keeps the upper triangle of a product and
mirrors it, as the library's symmetric epilogue does, and Y E and E Z are
mirrored in both forms as in the library): on a factor with eigenvalues
spread over [1e-8, 1] the two agree while the iteration is converging, but
once it has run long enough the mirrored coupling product lets rounding
errors grow until the iterates overflow, while the full product stays
finite.  The same happens on the GPU (config 4 with k = 15 and 20).
"""
import numpy as np


def _mirror(M):
    return np.triu(M) + np.triu(M, 1).T


def _ndb_pass(Y, iters, sym_p):
    n = Y.shape[0]
    I = np.eye(n, dtype=np.float32)
    Z = I.copy()
    for _ in range(iters):
        P = Z @ Y
        if sym_p:
            P = _mirror(P)
        E = (1.5 * I - 0.5 * P).astype(np.float32)
        Y, Z = _mirror(Y @ E).astype(np.float32), _mirror(E @ Z).astype(np.float32)
    return Y, Z


def _factor(n, seed):
    g = np.random.default_rng(seed)
    Q, _ = np.linalg.qr(g.standard_normal((n, n)))
    lam = 10.0 ** g.uniform(-8, 0, n)
    A = (Q * lam) @ Q.T
    return ((A + A.T) / (4 * lam.max())).astype(np.float32)  # scaled as by c = 2 lambda_max


def test_symmetric_coupling_agrees_early_and_overflows_late():
    As = _factor(128, 4)
    with np.errstate(all="ignore"):
        f8, m8 = _ndb_pass(As, 8, False), _ndb_pass(As, 8, True)
        f20, m20 = _ndb_pass(As, 20, False), _ndb_pass(As, 20, True)
    for a, b in zip(f8, m8):  # converging: the two forms agree to fp32 rounding
        assert np.linalg.norm(a - b) <= 1e-4 * np.linalg.norm(a)
    assert all(np.isfinite(m).all() for m in f20)
    assert not all(np.isfinite(m).all() for m in m20)
