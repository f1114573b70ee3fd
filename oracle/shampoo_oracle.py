"""Float64 CPU oracle for the Shampoo block-preconditioner update.

TEST INFRASTRUCTURE.  This module is the slow, plain reference that the HIP
path is checked against.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does.  It
shares no code with the HIP library and imports nothing from the package.

Everything is computed in float64 with numpy.  Matrix products use numpy's
`@` as a library primitive; there is no blocking, fusion or reordering beyond
what the formulas below state, so each function can be read against the
method description.

Sources, cited by page title and section:
  [DASH] "DASH: Faster Shampoo via Batched Block Preconditioning and
         Efficient Inverse-Root Solvers" -- the howistudyai.com explainer of
         the paper.  Sections are named as on that page ("Building blocks",
         "Step-by-step", "High-level flow", ...).  Its step-by-step list
         numbers every step "1."; steps are named here by their headings.
  [ABS]  the codewithpapers.app record of arXiv 2602.02016 (the abstract).
  [GVL]  Golub & Van Loan, Matrix Computations, the chapter on Jacobi
         methods for the symmetric eigenproblem (2x2 symmetric Schur
         decomposition, cyclic Jacobi).
  [GH]   Guo & Higham (2006), "A Schur-Newton method for the matrix p-th
         root and its inverse" -- the coupled Newton recurrence for A^{-1/p}.

Readings taken where the pages leave a step open are listed with each
function; the full list is in the design notes of the repository.

Status bits (per factor) mirror the ones the library reports:
  NONFINITE    = 1   a non-finite trace or eigenvalue estimate
  ZERO         = 2   trace of the factor is 0 (an all-zero history): X = I
  NONPOS_RQ    = 4   the spectral estimate is <= 0: X = I
  RESID_GROWTH = 8   a Newton residual rose above twice the smallest earlier
                     one of its pass (see residual_growth)
"""
from __future__ import annotations

import math

import numpy as np

NONFINITE = 1
ZERO = 2
NONPOS_RQ = 4
RESID_GROWTH = 8

F64 = np.float64


def _f64(a):
    return np.asarray(a, dtype=F64)


# ---------------------------------------------------------------------------
# Blocks and accumulation
# ---------------------------------------------------------------------------

def pad_block(g, B):
    """Zero-pad an r x c gradient block (r, c <= B) to B x B.

    Reading: the pages tile each layer gradient into B x B blocks and stack
    same-B blocks ([DASH] "Step-by-step", splitting into blocks and stacking);
    they do not say what happens to a partial edge block.  Here a partial
    block is the B x B block whose missing entries are zero, so it can share
    the stack.  Zero rows/columns only add directions with eigenvalue eps
    that never mix with the rest; U restricted to the real block is unchanged.
    """
    g = _f64(g)
    r, c = g.shape
    if r > B or c > B:
        raise ValueError("block larger than B")
    out = np.zeros((B, B), dtype=F64)
    out[:r, :c] = g
    return out


def accumulate(L, R, G, alpha, gamma):
    """One EMA step of the two Kronecker factors of a block.

    [DASH] "Step-by-step", building the preconditioners: the left factor is
    an exponential moving average of G G^T and the right one of G^T G:
        L <- alpha * L + gamma * G G^T,   R <- alpha * R + gamma * G^T G
    with alpha = beta and gamma = 1 - beta for the EMA (alpha = gamma = 1
    gives the plain running sum).  Reading: the state starts at zero and no
    bias correction is applied (the pages mention none).
    """
    G = _f64(G)
    return alpha * _f64(L) + gamma * (G @ G.T), alpha * _f64(R) + gamma * (G.T @ G)


def damping(F, eps_rel):
    """Trace and damping of a factor.

    [DASH] "Step-by-step", building the preconditioners: a multiple of the
    identity is added for stability.  Reading: eps = eps_rel * tr(F) / B,
    added to a working copy A = F + eps I (never stored into the EMA state).
    Returns (trace, eps).
    """
    F = _f64(F)
    tau = float(np.trace(F))
    return tau, eps_rel * tau / F.shape[0]


def damped(F, eps):
    F = _f64(F)
    return F + eps * np.eye(F.shape[0])


# ---------------------------------------------------------------------------
# Scaling
# ---------------------------------------------------------------------------

def frobenius_norm(A):
    """||A||_F -- the Frobenius scaling the pages compare against ([DASH]
    "Building blocks", Frobenius versus spectral scaling)."""
    A = _f64(A)
    return math.sqrt(float(np.sum(A * A)))


def power_iteration(A, V0, steps):
    """Multi-start power iteration for the largest eigenvalue of A.

    [DASH] "Building blocks", multi-power-iteration, and "Step-by-step",
    scaling each block: start from several random vectors at once, multiply
    by A repeatedly, keep the start whose Rayleigh quotient is largest.

    Readings: the r columns of V0 are the starts; each of `steps` rounds
    computes W = A V and normalises every column of W to unit 2-norm (a zero
    column stays zero); no orthogonalisation between columns.  After the
    last round one more product W = A V gives the Rayleigh quotients
    q_j = v_j^T w_j (the v_j have unit norm).  Returns (max_j q_j, q).
    """
    A = _f64(A)
    V = _f64(V0)
    for _ in range(steps):
        W = A @ V
        nrm = np.sqrt(np.sum(W * W, axis=0))
        inv = np.where(nrm > 0.0, 1.0 / np.where(nrm > 0.0, nrm, 1.0), 0.0)
        V = W * inv
    W = A @ V
    q = np.sum(V * W, axis=0)
    return float(np.max(q)), q


def scale_factor(F, eps_rel, mode, V0=None, steps=20, safety=2.0):
    """Trace, damping and the scale constant c of one factor.

    mode "power":     c = safety * lambda_est, lambda_est from
                      power_iteration(A, V0, steps).  [DASH] "Building
                      blocks": divide by about twice the estimate.  Reading:
                      exactly safety = 2.
    mode "frobenius": c = ||A||_F (it already bounds lambda_max).
    Degenerate factors (status bits above): trace 0 -> ZERO; estimate <= 0
    -> NONPOS_RQ; non-finite trace or estimate -> NONFINITE.
    Returns dict(trace, eps, lam, c, status).
    """
    F = _f64(F)
    tau, eps = damping(F, eps_rel)
    status = 0
    if not math.isfinite(tau):
        status |= NONFINITE
    elif tau == 0.0:
        status |= ZERO
    A = damped(F, eps)
    if mode == "power":
        if V0 is None:
            raise ValueError("power scaling needs start vectors")
        lam, _ = power_iteration(A, V0, steps)
        c = safety * lam
    elif mode == "frobenius":
        lam = frobenius_norm(A)
        c = lam
    else:
        raise ValueError(mode)
    if not math.isfinite(lam):
        status |= NONFINITE
    elif lam <= 0.0 and not (status & ZERO):
        status |= NONPOS_RQ
    return dict(trace=tau, eps=eps, lam=lam, c=c, status=status)


# ---------------------------------------------------------------------------
# Inverse-root solvers (matrix iterations, the pages' steps in order)
# ---------------------------------------------------------------------------

def newton_db_pass(Y0, iters):
    """One Newton-DB pass.

    [DASH] "Building blocks", Newton-DB, and "Step-by-step", solver (a):
    start with Y = Y0 and Z = I; each iteration forms E = (3I - Z Y)/2 and
    updates Y <- Y E and Z <- E Z.  Y tends to Y0^{1/2} and Z to Y0^{-1/2}
    for spectra inside (0, 3).  Returns (Y, Z, residuals) where
    residuals[i] = ||I - Z Y||_F at iteration i (before its update).
    """
    Y = _f64(Y0).copy()
    n = Y.shape[0]
    I = np.eye(n)
    Z = I.copy()
    res = []
    for _ in range(iters):
        P = Z @ Y
        res.append(math.sqrt(float(np.sum((I - P) ** 2))))
        E = 0.5 * (3.0 * I - P)
        Y, Z = Y @ E, E @ Z
    return Y, Z, res


def ndb_second_scale(iters):
    """Scale for the second pass of the Z-chained Newton-DB variant.

    Each first-pass factor E has eigenvalues in (1, 3/2] while the scaled
    spectrum lies in (0, 1], so Z_1 is bounded by (3/2)^iters; dividing by
    that bound puts the spectrum of Z_1 back inside (0, 1].
    """
    return 1.5 ** iters


def invroot_newton_db(A_s, iters, chaining="Y"):
    """A_s^{-1/4} by two chained Newton-DB passes of `iters` iterations each.

    [DASH] "Building blocks" says to chain two passes for the fourth root,
    and "Step-by-step", solver (a), to run the second pass on Y:
      chaining "Y" (the pages' reading): Y1 = pass(A_s).Y ~ A_s^{1/2};
                   X = pass(Y1).Z ~ Y1^{-1/2} = A_s^{-1/4}.
      chaining "Z" (a labelled variant, same number of products):
                   Z1 = pass(A_s).Z ~ A_s^{-1/2}; s2 = (3/2)^iters;
                   X = sqrt(s2) * pass(Z1 / s2).Y ~ A_s^{-1/4}.
    Reading: `iters` counts iterations per pass.
    Returns (X, residuals of both passes).
    """
    if chaining == "Y":
        Y1, _, r1 = newton_db_pass(A_s, iters)
        _, X, r2 = newton_db_pass(Y1, iters)
        return X, r1 + r2
    if chaining == "Z":
        _, Z1, r1 = newton_db_pass(A_s, iters)
        s2 = ndb_second_scale(iters)
        Y2, _, r2 = newton_db_pass(Z1 / s2, iters)
        return math.sqrt(s2) * Y2, r1 + r2
    raise ValueError(chaining)


def invroot_coupled_newton(A_s, p, iters):
    """A_s^{-1/p} by the coupled Newton iteration.

    [DASH] "Step-by-step", solver (b): X_k tends to A^{-1/p} with a coupled
    matrix M_k; each iteration forms C_k from M_k and sets X_{k+1} = X_k C_k
    and M_{k+1} = C_k^p M_k.  The page gives neither C_k nor the start; the
    reading follows [GH]: X_0 = I, M_0 = A_s, C_k = ((p+1) I - M_k) / p.
    The iteration converges for spectra inside (0, p+1).
    """
    return coupled_newton(A_s, p, iters)[0]


def coupled_newton(A_s, p, iters):
    """The coupled Newton iteration of invroot_coupled_newton with its
    residuals: returns (X, residuals), residuals[i] = ||I - M_i||_F at
    iteration i (before its update).  M_k tends to I as X_k tends to
    A_s^{-1/p} (M_k = X_k^p A_s in exact arithmetic), so the distance of M
    from I measures convergence the way ||I - Z Y||_F does for Newton-DB."""
    M = _f64(A_s).copy()
    n = M.shape[0]
    I = np.eye(n)
    X = I.copy()
    res = []
    for _ in range(iters):
        res.append(math.sqrt(float(np.sum((I - M) ** 2))))
        C = ((p + 1) * I - M) / p
        X = X @ C
        Cp = I.copy()
        for _ in range(p):
            Cp = Cp @ C
        M = Cp @ M
    return X, res


def chebyshev_coefficients(degree, p, delta):
    """Chebyshev interpolant of f(x) = x^{-1/p} on [delta, 1 + delta].

    [DASH] "Building blocks", Chebyshev, and "Step-by-step", solver (d):
    coefficients of a polynomial for the inverse root are fitted in advance
    on an interval, the spectrum is mapped into it, and the polynomial is
    evaluated with the Clenshaw recurrence.  Reading: the fit is the
    interpolant at the degree+1 first-kind Chebyshev nodes
        t_m = cos(pi (m + 1/2) / (degree + 1)),  x_m = delta + (1 + t_m) / 2,
        c_j = (2 / (degree + 1)) sum_m f(x_m) T_j(t_m),  c_0 halved,
    so that f(x) ~ sum_{j=0}^{degree} c_j T_j(2 (x - delta) - 1).
    """
    return chebyshev_interpolant(lambda t: (delta + 0.5 * (1.0 + t)) ** (-1.0 / p), degree)


def chebyshev_nodes(degree):
    """First-kind Chebyshev nodes t_m = cos(pi (m + 1/2) / (degree + 1))."""
    n = degree + 1
    return np.cos(math.pi * (np.arange(n, dtype=F64) + 0.5) / n)


def chebyshev_interpolant(fn, degree):
    """Coefficients c_0..c_degree of the polynomial sum_j c_j T_j(t) that
    interpolates fn at the first-kind nodes of [-1, 1] (c_0 halved)."""
    n = degree + 1
    theta = math.pi * (np.arange(n, dtype=F64) + 0.5) / n
    ft = np.asarray(fn(np.cos(theta)), dtype=F64)
    c = np.empty(n, dtype=F64)
    for j in range(n):
        c[j] = (2.0 / n) * float(np.sum(ft * np.cos(j * theta)))
    c[0] *= 0.5
    return c


def invroot_chebyshev(A_s, coeffs):
    """Evaluate sum_j c_j T_j(T) at the matrix T = 2 A_s - I by Clenshaw.

    [DASH] "Step-by-step", solver (d): the spectrum of the scaled factor
    (inside [0, 1]) is mapped onto the fitting interval; with the interval
    [delta, 1 + delta] the argument of the polynomial is 2 a - 1 for an
    eigenvalue a of A_s.  Clenshaw's recurrence:
        b_{d+1} = b_{d+2} = 0,
        b_j = c_j I + 2 T b_{j+1} - b_{j+2}   (j = d, ..., 1),
        result = c_0 I + T b_1 - b_2.
    """
    A_s = _f64(A_s)
    n = A_s.shape[0]
    I = np.eye(n)
    T = 2.0 * A_s - I
    d = len(coeffs) - 1
    b1 = np.zeros((n, n))
    b2 = np.zeros((n, n))
    for j in range(d, 0, -1):
        b1, b2 = coeffs[j] * I + 2.0 * (T @ b1) - b2, b1
    return coeffs[0] * I + T @ b1 - b2


# ---------------------------------------------------------------------------
# Full invroot stage and the preconditioned direction
# ---------------------------------------------------------------------------

def invroot(F, sc, method, iters=10, p=4, degree=24, delta=1e-12, chaining="Y"):
    """X = c^{-1/p} * g(A_s) for one factor, with A_s = (F + eps I) / c.

    `sc` is the dict from scale_factor.  method in {"ndb", "cn", "cheby",
    "exact"}.  Degenerate factors (ZERO or NONPOS_RQ) return X = I.  The
    final multiplication by c^{-1/p} undoes the scaling: (A/c)^{-1/p} =
    c^{1/p} A^{-1/p}.
    """
    F = _f64(F)
    n = F.shape[0]
    if sc["status"] & (ZERO | NONPOS_RQ):
        return np.eye(n)
    c = sc["c"]
    A_s = damped(F, sc["eps"]) / c
    if method == "ndb":
        if p == 2:  # one pass: Z tends to A_s^{-1/2}
            X = newton_db_pass(A_s, iters)[1]
        elif p == 4:
            X, _ = invroot_newton_db(A_s, iters, chaining)
        else:
            raise ValueError("Newton-DB gives p = 2 (one pass) or p = 4 (two chained passes)")
    elif method == "cn":
        X = invroot_coupled_newton(A_s, p, iters)
    elif method == "cheby":
        X = invroot_chebyshev(A_s, chebyshev_coefficients(degree, p, delta))
    elif method == "exact":
        X = invroot_exact(A_s, p)
    else:
        raise ValueError(method)
    return c ** (-1.0 / p) * X


def precondition(XL, G, XR):
    """U = X_L G X_R, the preconditioned block ([DASH] "High-level flow" and
    "Step-by-step", grafting: U is the preconditioned gradient)."""
    return _f64(XL) @ _f64(G) @ _f64(XR)


def adam_direction(m, v, g, beta1, beta2, eps, step):
    """Adam's moments and direction for one block (step >= 1).

    [DASH] "Step-by-step", grafting: the length of the update is borrowed
    from an Adam-like direction P.  Reading: plain Adam with bias
    correction,
        m <- beta1 m + (1 - beta1) g,   v <- beta2 v + (1 - beta2) g^2,
        P = (m / (1 - beta1^step)) / (sqrt(v / (1 - beta2^step)) + eps).
    Returns (m, v, P).
    """
    g = _f64(g)
    m = beta1 * _f64(m) + (1.0 - beta1) * g
    v = beta2 * _f64(v) + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** step)
    vhat = v / (1.0 - beta2 ** step)
    return m, v, mhat / (np.sqrt(vhat) + eps)


def graft_update(theta, m, v, g, U, lr, beta1, beta2, eps, step):
    """Grafted parameter update of one block.

    [DASH] "Step-by-step", grafting: with U the preconditioned gradient and
    P the Adam-like direction, s = ||P||_F / ||U||_F and theta <- theta -
    lr * s * U.  Readings: the norms are taken per block (U is formed per
    block); s = 0 when ||U||_F = 0 (then U = 0 and the step is zero anyway).
    Returns (theta, m, v, s).
    """
    m, v, P = adam_direction(m, v, g, beta1, beta2, eps, step)
    U = _f64(U)
    nu = math.sqrt(float(np.sum(U * U)))
    s = math.sqrt(float(np.sum(P * P))) / nu if nu > 0.0 else 0.0
    return _f64(theta) - lr * s * U, m, v, s


def residual_growth(residuals, per_pass, factor=2.0):
    """Whether a residual list shows growth: some residual of a pass exceeds
    `factor` times the smallest residual before it in the same pass.

    The pages report that some low-precision Newton iterations are unstable
    ([DASH] "Limitations": Newton-DB in FP16, coupled Newton in BF16;
    "Scoreboard with context": Frobenius-scaled Newton-DB at B = 2048) but
    give no detector.  Reading: in exact arithmetic ||I - Z Y||_F and
    ||I - M||_F never increase within a pass for spectra inside the
    convergence region (each eigenvalue's distance from 1 shrinks at every
    iteration), so a rise above twice an earlier value means rounding errors
    are being amplified.  `residuals` lists the passes one after another,
    `per_pass` entries each; non-finite entries compare like any other value
    (an infinite residual counts as growth, NaN never does).
    """
    res = [float(r) for r in residuals]
    for start in range(0, len(res), per_pass):
        lo = math.inf
        for r in res[start:start + per_pass]:
            if r > factor * lo:
                return True
            lo = min(lo, r)
    return False


def relative_frobenius(x, ref):
    """||x - ref||_F / ||ref||_F, the parity measure."""
    x = _f64(x)
    ref = _f64(ref)
    den = math.sqrt(float(np.sum(ref * ref)))
    num = math.sqrt(float(np.sum((x - ref) ** 2)))
    return num / den if den > 0 else num


def residual_fourth(X, A):
    """||X^4 A - I||_F in float64 (measurement of how close X is to A^{-1/4})."""
    X = _f64(X)
    X2 = X @ X
    R = X2 @ X2 @ _f64(A) - np.eye(X.shape[0])
    return math.sqrt(float(np.sum(R * R)))


# ---------------------------------------------------------------------------
# Jacobi eigendecomposition and exact inverse roots
# ---------------------------------------------------------------------------

def _sym_schur2(app, aqq, apq):
    """(c, s) of the rotation that diagonalises [[app, apq], [apq, aqq]]
    ([GVL], the 2x2 symmetric Schur decomposition): with
    tau = (aqq - app) / (2 apq) take the smaller root t of t^2 + 2 tau t - 1,
    then c = 1 / sqrt(1 + t^2), s = t c."""
    if apq == 0.0:
        return 1.0, 0.0
    tau = (aqq - app) / (2.0 * apq)
    if tau >= 0.0:
        t = 1.0 / (tau + math.sqrt(1.0 + tau * tau))
    else:
        t = -1.0 / (-tau + math.sqrt(1.0 + tau * tau))
    c = 1.0 / math.sqrt(1.0 + t * t)
    return c, t * c


def jacobi_eigh(A, tol=1e-15, max_sweeps=40):
    """Cyclic-by-row Jacobi eigendecomposition of a symmetric matrix ([GVL]).

    Sweeps over all pairs (p, q), p < q, applying the rotation J with
    J[p,p] = J[q,q] = c, J[p,q] = s, J[q,p] = -s as A <- J^T A J and
    accumulating V <- V J, until off(A) <= tol * ||A||_F.
    Returns (eigenvalues, V) with A = V diag(eigenvalues) V^T; eigenvalues
    in ascending order.  Intended for small blocks (Python loop over pairs).
    """
    A = _f64(A).copy()
    n = A.shape[0]
    if not np.allclose(A, A.T, rtol=0, atol=1e-12 * max(1.0, np.abs(A).max())):
        raise ValueError("jacobi_eigh needs a symmetric matrix")
    A = 0.5 * (A + A.T)
    V = np.eye(n)
    fro = math.sqrt(float(np.sum(A * A)))
    for _ in range(max_sweeps):
        offd = A - np.diag(np.diag(A))
        off = math.sqrt(float(np.sum(offd * offd)))
        if off <= tol * fro:
            break
        for p in range(n - 1):
            for q in range(p + 1, n):
                apq = A[p, q]
                if apq == 0.0:
                    continue
                c, s = _sym_schur2(A[p, p], A[q, q], apq)
                cp = A[:, p].copy()
                cq = A[:, q].copy()
                A[:, p] = c * cp - s * cq
                A[:, q] = s * cp + c * cq
                rp = A[p, :].copy()
                rq = A[q, :].copy()
                A[p, :] = c * rp - s * rq
                A[q, :] = s * rp + c * rq
                A[p, q] = 0.0
                A[q, p] = 0.0
                vp = V[:, p].copy()
                vq = V[:, q].copy()
                V[:, p] = c * vp - s * vq
                V[:, q] = s * vp + c * vq
    w = np.diag(A).copy()
    order = np.argsort(w)
    return w[order], V[:, order]


def invroot_exact(A, p):
    """A^{-1/p} = Q diag(lambda^{-1/p}) Q^T from the Jacobi decomposition.

    The eigen-decomposition route the pages keep as the accuracy reference
    ([DASH] "Step-by-step", solver (c)); needs a positive definite A.
    """
    w, Q = jacobi_eigh(A)
    if np.any(w <= 0.0):
        raise ValueError("exact inverse root needs a positive definite matrix")
    return (Q * (w ** (-1.0 / p))) @ Q.T


def spectral_apply(A, fn):
    """Q diag(fn(lambda)) Q^T for symmetric A via Jacobi (used to pin the
    matrix iterations: every iterate above is a polynomial in A)."""
    w, Q = jacobi_eigh(A)
    return (Q * fn(w)) @ Q.T


# Scalar forms of the recurrences (eigenvalue by eigenvalue) -------------

def ndb_pass_scalar(y0, iters):
    y = np.array(y0, dtype=F64)
    z = np.ones_like(y)
    for _ in range(iters):
        e = 0.5 * (3.0 - z * y)
        y, z = y * e, e * z
    return y, z


def ndb_scalar(a, iters, chaining="Y"):
    if chaining == "Y":
        y1, _ = ndb_pass_scalar(a, iters)
        return ndb_pass_scalar(y1, iters)[1]
    s2 = ndb_second_scale(iters)
    _, z1 = ndb_pass_scalar(a, iters)
    return math.sqrt(s2) * ndb_pass_scalar(z1 / s2, iters)[0]


def cn_scalar(a, p, iters):
    return cn_scalar_trace(a, p, iters)[0]


def cn_scalar_trace(a, p, iters):
    """Scalar coupled Newton: (x after `iters` iterations, [m_0, ..., m_{iters-1}])."""
    m = np.array(a, dtype=F64)
    x = np.ones_like(m)
    ms = []
    for _ in range(iters):
        ms.append(m.copy())
        q = ((p + 1) - m) / p
        x = x * q
        m = q ** p * m
    return x, ms


def cheby_scalar(a, coeffs):
    """sum_j c_j T_j(2a - 1) with T_j from the three-term recurrence
    T_0 = 1, T_1 = t, T_{j+1} = 2 t T_j - T_{j-1} (deliberately not Clenshaw)."""
    t = 2.0 * np.array(a, dtype=F64) - 1.0
    tp = np.ones_like(t)
    tc = t.copy()
    out = coeffs[0] * tp
    if len(coeffs) > 1:
        out = out + coeffs[1] * tc
    for j in range(2, len(coeffs)):
        tp, tc = tc, 2.0 * t * tc - tp
        out = out + coeffs[j] * tc
    return out


# ---------------------------------------------------------------------------
# One optimizer step for a stack of blocks (what the HIP path computes)
# ---------------------------------------------------------------------------

def shampoo_step(L, R, G, alpha, gamma, eps_rel, mode, V0L, V0R, method,
                 steps=20, safety=2.0, iters=10, p=4, degree=24, delta=1e-12,
                 chaining="Y"):
    """Full hot path for one block: accumulate, scale, inverse roots, U.

    Returns dict(L, R, XL, XR, U, scL, scR).  L and R are the EMA states
    before the step (zeros for a fresh optimizer); G is the B x B
    (zero-padded) gradient block.
    """
    Ln, Rn = accumulate(L, R, G, alpha, gamma)
    scL = scale_factor(Ln, eps_rel, mode, V0L, steps, safety)
    scR = scale_factor(Rn, eps_rel, mode, V0R, steps, safety)
    kw = dict(iters=iters, p=p, degree=degree, delta=delta, chaining=chaining)
    XL = invroot(Ln, scL, method, **kw)
    XR = invroot(Rn, scR, method, **kw)
    return dict(L=Ln, R=Rn, XL=XL, XR=XR, U=precondition(XL, G, XR), scL=scL, scR=scR)



def shampoo_run(grads, alpha, gamma, eps_rel, mode, V0L, V0R, method, update_every=1,
                steps=20, safety=2.0, iters=10, p=4, degree=24, delta=1e-12, chaining="Y"):
    """Several optimizer steps on one block with the roots refreshed every
    `update_every` steps and cached in between.

    [DASH] "Scoreboard with context" quotes runs at update frequency f = 10,
    where only every f-th step pays for the roots and the steps between are
    cheap; "Required resources" keeps the inverse roots cached in memory.
    Reading: the factors are accumulated at every step; the scale and the
    roots are recomputed at steps 1, 1 + f, 1 + 2 f, ... (counting from 1)
    from the factors of that step; every step preconditions its own gradient
    with the most recent roots.  Starts from zero factors.

    Returns a list of dicts (L, R, XL, XR, U, refreshed) per step.
    """
    n = grads[0].shape[0]
    L = np.zeros((n, n))
    R = np.zeros((n, n))
    kw = dict(iters=iters, p=p, degree=degree, delta=delta, chaining=chaining)
    out = []
    XL = XR = None
    for t, G in enumerate(grads):
        L, R = accumulate(L, R, G, alpha, gamma)
        refreshed = t % update_every == 0
        if refreshed:
            XL = invroot(L, scale_factor(L, eps_rel, mode, V0L, steps, safety), method, **kw)
            XR = invroot(R, scale_factor(R, eps_rel, mode, V0R, steps, safety), method, **kw)
        out.append(dict(L=L, R=R, XL=XL, XR=XR, U=precondition(XL, G, XR), refreshed=refreshed))
    return out