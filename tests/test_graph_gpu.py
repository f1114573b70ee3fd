"""A whole optimizer step captured as HIP graphs (ShampooBlocks.capture) and
replayed: every replay, with eager work and synchronisations in between, must
give the bits of the same step run eagerly.  The library enqueues only kernel
launches (no memset, no allocation once the workspaces are reserved)."""
import numpy as np
import pytest
import torch

from inverse_root_preconditioning_amd import capi
from inverse_root_preconditioning_amd import pipeline as PL
from inverse_root_preconditioning_amd import workloads as W

from gpu_helpers import dev, host, report

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    capi.load()


def _state(cfg, n, V0):
    st = PL.ShampooBlocks(cfg, n)
    st.set_start_vectors(V0)
    return st


@pytest.mark.parametrize("update_every,variant", [(1, capi.NDB_Z), (2, capi.NDB_Z), (1, capi.CN)])
def test_captured_step_replays_match_eager(update_every, variant):
    B = 256
    grads = [W.config2_gradient(t) for t in range(1, 6)]
    cfg = PL.StepConfig(B=B, beta=0.95, eps_rel=1e-12, variant=variant, iters=10, update_every=update_every)
    g_e, g_g = dev(grads[0]), dev(grads[0])
    u_e, u_g = torch.empty_like(g_e), torch.empty_like(g_g)
    tab = {k: (PL.BlockTable.from_layers([g], B), PL.BlockTable.from_layers([u], B))
           for k, g, u in (("e", g_e, u_e), ("g", g_g, u_g))}
    n = tab["e"][0].n
    V0 = dev(W.start_vectors(2, 2 * n, B))
    eager, graphed = _state(cfg, n, V0), _state(cfg, n, V0)
    sg = graphed.capture(*tab["g"])
    assert len(sg.graphs) == (1 if update_every == 1 else 2)
    for t, G in enumerate(grads):
        g_e.copy_(torch.from_numpy(G))
        g_g.copy_(torch.from_numpy(G))
        eager.step(*tab["e"])          # the program's own eager work between replays
        torch.cuda.synchronize()
        sg.replay()
        torch.cuda.synchronize()
        assert graphed.t == eager.t == t + 1
        for a, b, name in ((u_g, u_e, "U"), (graphed.factors, eager.factors, "factors"),
                           (graphed.roots, eager.roots, "roots"), (graphed.status, eager.status, "status")):
            assert np.array_equal(host(a), host(b)), (t, name)
        assert np.all(np.isfinite(host(u_g)))
    report("graph_replay", update_every=update_every, variant=variant, steps=len(grads), ok=True)
