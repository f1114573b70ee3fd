"""Fault-injection inputs and checkpoint/resume of the whole step, through the
C ABI, against the float64 oracle.

* A NaN inside one gradient block, a gradient block with an entry of 1e38
  (its Gram factors overflow fp32) and blocks scaled by 1e15 and 1e-15 share
  one launch with ordinary blocks: the bad blocks are flagged NONFINITE, the
  scaled ones and every ordinary block still match the oracle, and nothing
  leaks from one block into another.
* Five straight steps equal three steps, a save and load of the optimizer
  state, and two more steps, bit for bit (the kernels are deterministic).
"""
import io

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


B = 256
NAN_BLOCK, BIG_BLOCK, UP_BLOCK, DOWN_BLOCK = 6, 9, 3, 12


def poisoned_gradient():
    """Config 2's first gradient (1024 x 1024, 4 x 4 blocks of 256) with a NaN
    in block 6, an entry of 1e38 in block 9, block 3 scaled by 1e15 and block
    12 by 1e-15."""
    G = W.config2_gradient(1).copy()

    def blk(i):
        return G[(i // 4) * B:(i // 4 + 1) * B, (i % 4) * B:(i % 4 + 1) * B]

    blk(NAN_BLOCK)[44, 188] = np.nan
    blk(BIG_BLOCK)[10, 20] = np.float32(1e38)
    blk(UP_BLOCK)[:] *= np.float32(1e15)
    blk(DOWN_BLOCK)[:] *= np.float32(1e-15)
    return G


@pytest.mark.parametrize("variant", [capi.NDB_Z, capi.CN])
def test_bad_gradient_blocks_are_flagged_and_contained(variant):
    G = poisoned_gradient()
    k = 10
    gt = dev(G)
    table = PL.BlockTable.from_layers([gt], B)
    n = table.n
    cfg = PL.StepConfig(B=B, beta=0.95, eps_rel=1e-12, variant=variant, iters=k)
    state = PL.ShampooBlocks(cfg, n)
    V0 = W.start_vectors(2, 2 * n, B)
    state.set_start_vectors(dev(V0))
    U = torch.full_like(gt, 7.0)
    state.step(table, PL.BlockTable.from_layers([U], B))
    F, X, Uh, st = host(state.factors), host(state.roots), host(U), host(state.status)
    method = "ndb" if variant == capi.NDB_Z else "cn"
    ex = eu = 0.0
    for i in range(n):
        r0, c0 = (i // 4) * B, (i % 4) * B
        g = G[r0:r0 + B, c0:c0 + B]
        if i == NAN_BLOCK:
            # the NaN reaches only row/column 44 of L and row/column 188 of R
            L, R = F[i], F[n + i]
            assert np.isnan(L[44, :]).all() and np.isnan(L[:, 44]).all()
            assert np.isfinite(np.delete(np.delete(L, 44, 0), 44, 1)).all()
            assert np.isnan(R[188, :]).all() and np.isfinite(np.delete(np.delete(R, 188, 0), 188, 1)).all()
        if i in (NAN_BLOCK, BIG_BLOCK):
            # a NaN, or a Gram factor beyond fp32's range (1e76 on the diagonal): flagged, values propagate
            assert st[i] & capi.BLK_NONFINITE and st[n + i] & capi.BLK_NONFINITE, (i, st[i], st[n + i])
            assert not np.isfinite(Uh[r0:r0 + B, c0:c0 + B]).all()
            continue
        assert st[i] == 0 and st[n + i] == 0, (i, st[i], st[n + i])
        L, R = O.accumulate(np.zeros((B, B)), np.zeros((B, B)), g, 0.95, 0.05)
        xs = []
        for j, Fo in ((i, L), (n + i, R)):
            so = O.scale_factor(Fo, 1e-12, "power", V0[j], 20, 2.0)
            assert so["status"] == 0
            xo = O.invroot(Fo, so, method, iters=k, chaining="Z")
            ex = max(ex, O.relative_frobenius(X[j], xo))
            xs.append(xo)
        eu = max(eu, O.relative_frobenius(Uh[r0:r0 + B, c0:c0 + B], O.precondition(xs[0], g, xs[1])))
    report("poisoned_blocks", variant=variant, root_err=ex, U_err=eu)
    assert ex <= TOL_F32 and eu <= TOL_F32, (ex, eu)
    # U does not depend on the scale of G: the 1e15 and 1e-15 blocks give the unscaled block's U
    G0 = W.config2_gradient(1)
    ref = torch.empty_like(gt)
    s2 = PL.ShampooBlocks(cfg, n)
    s2.set_start_vectors(dev(V0))
    gt.copy_(torch.from_numpy(G0))
    s2.step(table, PL.BlockTable.from_layers([ref], B))
    R0 = host(ref)
    for i in (UP_BLOCK, DOWN_BLOCK):
        r0, c0 = (i // 4) * B, (i % 4) * B
        e = O.relative_frobenius(Uh[r0:r0 + B, c0:c0 + B], R0[r0:r0 + B, c0:c0 + B])
        assert e <= TOL_F32, (i, e)


@pytest.mark.parametrize("update_every", [1, 2])
def test_checkpoint_resume_is_bitwise(update_every):
    """Config 2's five steps straight, against three steps, torch.save of the
    state, a fresh optimizer loaded from it (weights_only=True), and two more
    steps.  With update_every = 2 the roots cached at step 3 carry step 4."""
    grads = [W.config2_gradient(t) for t in range(1, 6)]
    cfg = PL.StepConfig(B=B, beta=0.95, eps_rel=1e-12, variant=capi.NDB_Z, iters=10, update_every=update_every)
    gt = dev(grads[0])
    table = PL.BlockTable.from_layers([gt], B)
    n = table.n
    V0 = dev(W.start_vectors(2, 2 * n, B))
    U = torch.empty_like(gt)
    utable = PL.BlockTable.from_layers([U], B)

    def run(state, steps):
        outs = []
        for t in steps:
            gt.copy_(torch.from_numpy(grads[t]))
            state.step(table, utable)
            outs.append((host(U).copy(), host(state.factors).copy(), host(state.roots).copy()))
        return outs

    straight = PL.ShampooBlocks(cfg, n)
    straight.set_start_vectors(V0)
    full = run(straight, range(5))

    first = PL.ShampooBlocks(cfg, n)
    first.set_start_vectors(V0)
    run(first, range(3))
    buf = io.BytesIO()
    torch.save(first.state_dict(), buf)
    del first
    buf.seek(0)
    resumed = PL.ShampooBlocks(cfg, n)
    resumed.load_state_dict(torch.load(buf, weights_only=True, map_location="cuda"))
    resumed.set_start_vectors(V0)
    assert resumed.t == 3 and resumed.refresh_due == (3 % update_every == 0)
    tail = run(resumed, range(3, 5))
    for (ua, fa, xa), (ub, fb, xb) in zip(full[3:], tail):
        assert np.array_equal(ua, ub) and np.array_equal(fa, fb) and np.array_equal(xa, xb)
    report("checkpoint_resume", update_every=update_every, ok=True)


_LOAD_FIRST = r"""
import sys
sys.path.insert(0, sys.argv[1])
from inverse_root_preconditioning_amd import capi
capi.load()                      # the library before any explicit torch import
import torch
from inverse_root_preconditioning_amd import pipeline as PL
g = torch.randn((2, 64, 64), device="cuda")
F = torch.zeros((4, 64, 64), device="cuda")
PL.accumulate(PL.BlockTable.from_stack(g), F, 0.0, 1.0)
torch.cuda.synchronize()
ref = torch.cat([g @ g.transpose(1, 2), g.transpose(1, 2) @ g])
err = ((F - ref).norm() / ref.norm()).item()
print("ok" if err < 1e-5 else f"err {err}")
"""


def test_library_loaded_before_torch():
    """Loading the library before PyTorch must still bind it to PyTorch's HIP
    runtime (a second runtime in the process fails every launch)."""
    import subprocess
    import sys
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", _LOAD_FIRST, root], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip().splitlines()[-1] == "ok", out.stdout
