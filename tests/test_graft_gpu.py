"""Parity of the grafted parameter update (Adam's magnitude, Shampoo's
direction) with the float64 oracle over three steps, on ragged blocks."""
import numpy as np
import pytest
import torch

from oracle import shampoo_oracle as O
from inverse_root_preconditioning_amd import capi
from inverse_root_preconditioning_amd import pipeline as PL
from inverse_root_preconditioning_amd import workloads as W

from gpu_helpers import TOL_F32, dev, host, report

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    capi.load()


def blocks_of(shape, B):
    m, n = shape
    return [(r0, c0, min(B, m - r0), min(B, n - c0)) for r0 in range(0, m, B) for c0 in range(0, n, B)]


@pytest.mark.parametrize("B", [128, 256])
def test_graft_update_three_steps(B):
    shape = (300, 520)
    lr, b1, b2, eps = 1e-2, 0.9, 0.95, 1e-8
    theta = W.ragged_gradients(300 + B, [shape], 1.0)[0]
    th, mt, vt = dev(theta), torch.zeros(shape, device="cuda"), torch.zeros(shape, device="cuda")
    g_t, u_t = torch.empty(shape, device="cuda"), torch.empty(shape, device="cuda")
    tabs = [PL.BlockTable.from_layers([t], B) for t in (g_t, u_t, th, mt, vt)]
    n = tabs[0].n
    s_out = torch.zeros(n, device="cuda")
    theta64, m64, v64 = theta.astype(np.float64), np.zeros(shape), np.zeros(shape)
    for step in (1, 2, 3):
        g = W.ragged_gradients(400 + 10 * B + step, [shape], 0.02)[0]
        U = W.ragged_gradients(500 + 10 * B + step, [shape], 1.0)[0]
        if step == 3:
            U[:B, :B] = 0.0  # a zero update block: s = 0, theta unchanged there
        g_t.copy_(torch.from_numpy(g))
        u_t.copy_(torch.from_numpy(U))
        PL.graft_update(*tabs, lr, b1, b2, eps, step, s_out)
        th_h, m_h, v_h, s_h = host(th), host(mt), host(vt), host(s_out)
        errs = {"theta_step": 0.0, "m": 0.0, "v": 0.0, "s": 0.0}
        for i, (r0, c0, rows, cols) in enumerate(blocks_of(shape, B)):
            sl = (slice(r0, r0 + rows), slice(c0, c0 + cols))
            prev = theta64[sl].copy()
            nt, nm, nv, s = O.graft_update(prev, m64[sl], v64[sl], g[sl], U[sl], lr, b1, b2, eps, step)
            theta64[sl], m64[sl], v64[sl] = nt, nm, nv
            errs["theta_step"] = max(errs["theta_step"], O.relative_frobenius(th_h[sl] - prev, nt - prev)
                                     if s > 0 else float(np.abs(th_h[sl] - prev).max()))
            errs["m"] = max(errs["m"], O.relative_frobenius(m_h[sl], nm))
            errs["v"] = max(errs["v"], O.relative_frobenius(v_h[sl], nv))
            errs["s"] = max(errs["s"], abs(s_h[i] - s) / s if s > 0 else abs(s_h[i]))
            theta64[sl] = th_h[sl]  # carry the GPU's fp32 parameters, the oracle's own moments
        report("graft", B=B, step=step, **errs)
        assert errs["m"] <= 1e-6 and errs["v"] <= 1e-6 and errs["s"] <= 1e-5
        assert errs["theta_step"] <= TOL_F32
