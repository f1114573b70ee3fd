"""The allocation-free grafting entry point (shampoo_graft_update_noalloc)
against the workspace one (shampoo_graft_update), both through the C ABI on
identical inputs: two calls in a row, the second on a smaller input, must give
the same parameters, moments and grafting scales bit for bit (the same
kernels run in the same order; only where the partial norms live differs)."""
import numpy as np
import pytest
import torch

from inverse_root_preconditioning_amd import capi
from inverse_root_preconditioning_amd import pipeline as PL
from inverse_root_preconditioning_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    capi.load()


def _state(key, shape):
    theta, g, u = W.ragged_gradients(key, [shape, shape, shape], 1.0)
    m = np.abs(W.ragged_gradients(key + 1, [shape], 0.01)[0])
    v = np.abs(W.ragged_gradients(key + 2, [shape], 0.001)[0])
    return [torch.from_numpy(a).cuda() for a in (g, u, theta, m, v)]


def _run(entry, tensors, B, step):
    """Returns (theta, m, v, s) after one grafted update through `entry`."""
    g, u, theta, m, v = [t.clone() for t in tensors]
    tabs = [PL.BlockTable.from_layers([t], B) for t in (g, u, theta, m, v)]
    n = tabs[0].n
    s = torch.full((n,), -1.0, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    args = [t.ptr for t in tabs] + [n, B, 1e-2, 0.9, 0.95, 1e-8, step, s.data_ptr()]
    if entry == "noalloc":
        rc = capi.shampoo_graft_update_noalloc(*args, stream)
    else:
        ws = PL.Workspace()
        wp, wb = ws.get(capi.shampoo_workspace_bytes(capi.OP_GRAFT, n, B, 0, capi.F32))
        rc = capi.shampoo_graft_update(*args, wp, wb, stream)
    assert rc == capi.OK, capi.strerror(rc)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (theta, m, v, s)], n


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    # first call: 3 x 5 blocks of 256 (ragged edges); second: fewer, smaller blocks at B = 128
    for key, shape, B, step in ((11, (700, 1200), 256, 3), (21, (200, 300), 128, 1)):
        tensors = _state(key, shape)
        print(f"noalloc case: shape={shape} B={B} step={step}", flush=True)
        ref, n = _run("workspace", tensors, B, step)
        out, n2 = _run("noalloc", tensors, B, step)
        assert n == n2
        for name, a, b in zip(("theta", "m", "v", "s"), out, ref):
            assert np.array_equal(a, b), name
        assert np.all(ref[3] > 0) and np.all(np.isfinite(ref[0]))
        assert not np.array_equal(ref[0], tensors[2].cpu().numpy())  # the update did move theta


def test_noalloc_rejects_problems_beyond_its_scratch():
    B = 1024                      # 16 chunks per block: 128 bytes of partial norms per block
    limit = capi.NOALLOC_SCRATCH_BYTES // 128
    fake = 0x10000                # never dereferenced: the call returns before any launch
    args = [fake] * 5
    rc = capi.shampoo_graft_update_noalloc(*args, limit + 1, B, 1e-2, 0.9, 0.95, 1e-8, 1, 0, 0)
    assert rc == capi.ESCRATCH
    assert "static scratch" in capi.strerror(rc)
