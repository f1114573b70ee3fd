"""Torch-tensor layer over the C ABI: descriptor tables, workspaces and the
per-step driver.  PyTorch provides device memory and the stream; all the
arithmetic runs in the HIP library (see capi).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from . import capi

F32 = capi.F32
BF16_IN = capi.BF16_IN


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t):
    return 0 if t is None else t.data_ptr()


def _check_f32_cuda(t, name, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not (t.is_cuda and t.dtype == torch.float32 and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous float32 CUDA tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_scale_status(scale, status, nf):
    """scale: [nf, 4] float32 (c, eps, lambda, trace); status: [nf] int32."""
    _check_f32_cuda(scale, "scale", (nf, 4))
    if status is None:
        raise ValueError("status is required")
    if not (status.is_cuda and status.dtype == torch.int32 and status.is_contiguous()):
        raise ValueError("status must be a contiguous int32 CUDA tensor")
    if tuple(status.shape) != (nf,):
        raise ValueError(f"status has shape {tuple(status.shape)}, expected {(nf,)}")


def residual_columns(p, variant, iters):
    """Columns of resid_out for shampoo_invroot_newton: one per iteration of
    each pass (Newton-DB for p = 4 runs two passes, p = 2 and coupled Newton one)."""
    base = variant & 0xff
    passes = 1 if (p == 2 or base in (capi.CN, capi.CN_F16)) else 2
    return passes * iters


class BlockTable:
    """Device array of shampoo_block descriptors (24 bytes each) plus the
    tensors it points into (kept alive with the table)."""

    def __init__(self, entries, B, device=None):
        n = len(entries)
        arr = np.zeros((max(n, 1), 3), dtype=np.int64)
        keep = []
        for i, (t, r0, c0, rows, cols) in enumerate(entries):
            if t.dtype != torch.float32 or t.dim() != 2 or t.stride(1) != 1:
                raise ValueError("blocks must come from row-major float32 2D tensors")
            if not (0 <= rows <= B and 0 <= cols <= B):
                raise ValueError("block larger than B")
            if r0 < 0 or c0 < 0 or r0 + rows > t.shape[0] or c0 + cols > t.shape[1]:
                raise ValueError("block outside its tensor")
            ld = t.stride(0)
            arr[i, 0] = t.data_ptr() + 4 * (r0 * ld + c0)
            arr[i, 1] = ld
            arr[i, 2] = int(rows) | (int(cols) << 32)
            keep.append(t)
        self.n = n
        self.B = B
        self._keep = keep
        dev = device if device is not None else (entries[0][0].device if n else torch.device("cuda"))
        self.tensor = torch.from_numpy(arr).to(dev)

    @property
    def ptr(self):
        return self.tensor.data_ptr()

    @classmethod
    def from_stack(cls, stack):
        """One full B x B block per item of a [n, B, B] tensor."""
        n, B, _ = stack.shape
        return cls([(stack[i], 0, 0, B, B) for i in range(n)], B, stack.device)

    @classmethod
    def from_layers(cls, tensors, B):
        """Row-major B x B tiling of each 2D tensor, tensors in order (edge
        blocks may be partial)."""
        entries = []
        for t in tensors:
            m, n = t.shape
            for r0 in range(0, m, B):
                for c0 in range(0, n, B):
                    entries.append((t, r0, c0, min(B, m - r0), min(B, n - c0)))
        return cls(entries, B, tensors[0].device if tensors else None)


class Workspace:
    """Grow-only scratch buffer (uint8 CUDA tensor)."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes):
        nbytes = max(int(nbytes), 256)
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf.data_ptr(), self.buf.numel()


def accumulate(table, factors, alpha, gamma, prec=F32, ws=None, stream=None):
    n, B = table.n, table.B
    _check_f32_cuda(factors, "factors", (2 * n, B, B))
    ws = ws or Workspace(factors.device)
    need = capi.shampoo_workspace_bytes(capi.OP_ACCUMULATE, n, B, 0, prec)
    wp, wb = ws.get(need) if need else (0, 0)
    capi.check(capi.shampoo_accumulate(table.ptr, n, B, factors.data_ptr(), alpha, gamma, prec, wp, wb,
                                       _stream(stream)), "shampoo_accumulate")


def new_scale(nf, device):
    """(scale [nf, 4] float32: c, eps, lambda, trace; status [nf] int32)."""
    return (torch.zeros((nf, 4), dtype=torch.float32, device=device),
            torch.zeros((nf,), dtype=torch.int32, device=device))


def scale_power(factors, eps_rel, mode, v0, steps, safety, scale, status, ws=None, stream=None):
    _check_f32_cuda(factors, "factors")
    nf, B, _ = factors.shape
    _check_scale_status(scale, status, nf)
    r = 0
    if mode == capi.SCALE_POWER:
        _check_f32_cuda(v0, "v0")
        if v0.shape[0] != nf or v0.shape[1] != B:
            raise ValueError("v0 must be [nfactors, B, r]")
        r = v0.shape[2]
    ws = ws or Workspace(factors.device)
    wp, wb = ws.get(capi.shampoo_workspace_bytes(capi.OP_SCALE, nf, B, 0, F32))
    capi.check(capi.shampoo_scale_power(factors.data_ptr(), nf, B, eps_rel, mode, _ptr(v0), r, steps, safety,
                                        scale.data_ptr(), status.data_ptr(), wp, wb, _stream(stream)),
               "shampoo_scale_power")


def invroot_newton(factors, scale, p, variant, iters, x_out, status, resid_out=None, ws=None, stream=None):
    _check_f32_cuda(factors, "factors")
    nf, B, _ = factors.shape
    _check_f32_cuda(x_out, "x_out", factors.shape)
    _check_scale_status(scale, status, nf)
    if resid_out is not None:
        _check_f32_cuda(resid_out, "resid_out", (nf, residual_columns(p, variant, iters)))
    ws = ws or Workspace(factors.device)
    wp, wb = ws.get(capi.shampoo_workspace_bytes(capi.OP_NEWTON, nf, B, variant, F32))
    capi.check(capi.shampoo_invroot_newton(factors.data_ptr(), scale.data_ptr(), nf, B, p, variant, iters,
                                           x_out.data_ptr(), _ptr(resid_out), status.data_ptr(), wp, wb,
                                           _stream(stream)), "shampoo_invroot_newton")


def invroot_cheby(factors, scale, p, degree, interval_eps, prec, x_out, status, ws=None, stream=None):
    _check_f32_cuda(factors, "factors")
    nf, B, _ = factors.shape
    _check_f32_cuda(x_out, "x_out", factors.shape)
    _check_scale_status(scale, status, nf)
    ws = ws or Workspace(factors.device)
    wp, wb = ws.get(capi.shampoo_workspace_bytes(capi.OP_CHEBY, nf, B, degree, prec))
    capi.check(capi.shampoo_invroot_cheby(factors.data_ptr(), scale.data_ptr(), nf, B, p, degree, interval_eps,
                                          prec, x_out.data_ptr(), status.data_ptr(), wp, wb, _stream(stream)),
               "shampoo_invroot_cheby")


def precondition(x_roots, g_table, u_table, prec=F32, ws=None, stream=None):
    n, B = g_table.n, g_table.B
    _check_f32_cuda(x_roots, "x_roots", (2 * n, B, B))
    if u_table.n != n:
        raise ValueError("output table size differs from the gradient table")
    ws = ws or Workspace(x_roots.device)
    need = capi.shampoo_workspace_bytes(capi.OP_PRECONDITION, n, B, 0, prec)
    wp, wb = ws.get(need)
    capi.check(capi.shampoo_precondition(x_roots.data_ptr(), g_table.ptr, n, B, u_table.ptr, prec, wp, wb,
                                         _stream(stream)), "shampoo_precondition")


def graft_update(g_table, u_table, p_table, m_table, v_table, lr, beta1, beta2, eps, step, scale_out=None,
                 ws=None, stream=None):
    """theta <- theta - lr (||P||_F / ||U||_F) U per block, P Adam's direction (m, v updated)."""
    n, B = g_table.n, g_table.B
    for t in (u_table, p_table, m_table, v_table):
        if t.n != n or t.B != B:
            raise ValueError("descriptor tables differ in size")
    ws = ws or Workspace(g_table.tensor.device)
    wp, wb = ws.get(capi.shampoo_workspace_bytes(capi.OP_GRAFT, n, B, 0, F32))
    capi.check(capi.shampoo_graft_update(g_table.ptr, u_table.ptr, p_table.ptr, m_table.ptr, v_table.ptr, n, B,
                                         lr, beta1, beta2, eps, step, _ptr(scale_out), wp, wb, _stream(stream)),
               "shampoo_graft_update")


@dataclass
class StepConfig:
    """One optimizer step of the block preconditioner (defaults: the pages'
    Newton-DB with power-iteration scaling)."""
    B: int
    beta: float = 0.95          # EMA factor: alpha = beta, gamma = 1 - beta
    eps_rel: float = 1e-12      # damping eps = eps_rel tr(F) / B
    scale_mode: int = capi.SCALE_POWER
    pi_steps: int = 20
    pi_starts: int = 32
    safety: float = 2.0
    solver: str = "newton"      # "newton" or "cheby"
    variant: int = capi.NDB
    iters: int = 10
    p: int = 4
    degree: int = 24
    interval_eps: float = 1e-12
    prec: int = F32
    keep_resid: bool = False
    update_every: int = 1       # roots refreshed at steps 1, 1 + f, 1 + 2f, ...; cached in between


@dataclass
class ShampooBlocks:
    """State and workspaces for a fixed set of gradient blocks.

    The factors are accumulated at every step.  With update_every = f > 1 the
    scale and the inverse roots are recomputed only at steps 1, 1 + f,
    1 + 2f, ... (the pages' update frequency) and the cached roots
    precondition the steps in between.  `t` counts the steps taken."""
    cfg: StepConfig
    nblocks: int
    device: object = "cuda"
    factors: torch.Tensor = field(init=False)
    roots: torch.Tensor = field(init=False)

    def __post_init__(self):
        B, n, dev = self.cfg.B, self.nblocks, self.device
        self.factors = torch.zeros((2 * n, B, B), dtype=torch.float32, device=dev)
        self.roots = torch.empty((2 * n, B, B), dtype=torch.float32, device=dev)
        self.scale, self.status = new_scale(2 * n, dev)
        self.resid = None
        if self.cfg.keep_resid and self.cfg.solver == "newton":
            cols = residual_columns(self.cfg.p, self.cfg.variant, self.cfg.iters)
            self.resid = torch.zeros((2 * n, cols), dtype=torch.float32, device=dev)
        self.ws = {k: Workspace(dev) for k in ("acc", "scale", "root", "pre")}
        self.v0 = None
        if self.cfg.update_every < 1:
            raise ValueError("update_every must be >= 1")
        self.t = 0

    def state_dict(self):
        """The optimizer state needed to resume bit for bit: the EMA factors,
        the cached roots with their scale records and status, and the step
        count.  Tensors are returned as they are (device tensors); save them
        with torch.save and load with torch.load(..., weights_only=True).
        The power-iteration start vectors are the caller's input and are set
        again with set_start_vectors after a restore."""
        return {"factors": self.factors, "roots": self.roots, "scale": self.scale, "status": self.status,
                "t": int(self.t), "B": int(self.cfg.B), "nblocks": int(self.nblocks)}

    def load_state_dict(self, sd):
        """Restore a state_dict() of a ShampooBlocks with the same B and block count."""
        if int(sd["B"]) != self.cfg.B or int(sd["nblocks"]) != self.nblocks:
            raise ValueError("state was saved for a different block size or block count")
        for name in ("factors", "roots", "scale", "status"):
            dst = getattr(self, name)
            src = sd[name]
            if tuple(src.shape) != tuple(dst.shape) or src.dtype != dst.dtype:
                raise ValueError(f"{name}: saved {tuple(src.shape)} {src.dtype}, expected "
                                 f"{tuple(dst.shape)} {dst.dtype}")
            dst.copy_(src)
        self.t = int(sd["t"])

    def set_start_vectors(self, v0):
        _check_f32_cuda(v0, "v0", (2 * self.nblocks, self.cfg.B, v0.shape[2]))
        self.v0 = v0

    @property
    def refresh_due(self):
        """Whether the next step recomputes the roots."""
        return self.t % self.cfg.update_every == 0

    def step(self, g_table, u_table, stream=None):
        self._enqueue(g_table, u_table, self.refresh_due, stream)
        self.t += 1

    def _enqueue(self, g_table, u_table, refresh, stream=None):
        """Enqueue one step's launches (no host-side state changes)."""
        c = self.cfg
        accumulate(g_table, self.factors, c.beta, 1.0 - c.beta, c.prec, self.ws["acc"], stream)
        if refresh:
            self.update_roots(stream)
        precondition(self.roots, g_table, u_table, c.prec, self.ws["pre"], stream)

    def reserve(self):
        """Allocate every workspace a step needs, so that later steps allocate
        nothing (required before capture)."""
        c, n, B = self.cfg, self.nblocks, self.cfg.B
        nf = 2 * n
        self.ws["acc"].get(capi.shampoo_workspace_bytes(capi.OP_ACCUMULATE, n, B, 0, c.prec))
        self.ws["scale"].get(capi.shampoo_workspace_bytes(capi.OP_SCALE, nf, B, 0, F32))
        if c.solver == "newton":
            self.ws["root"].get(capi.shampoo_workspace_bytes(capi.OP_NEWTON, nf, B, c.variant, F32))
        else:
            self.ws["root"].get(capi.shampoo_workspace_bytes(capi.OP_CHEBY, nf, B, c.degree, c.prec))
        self.ws["pre"].get(capi.shampoo_workspace_bytes(capi.OP_PRECONDITION, n, B, 0, c.prec))

    def capture(self, g_table, u_table):
        """Capture one step over these descriptor tables as HIP graphs (one with
        a root refresh and, for update_every > 1, one with cached roots) and
        return a StepGraph whose replay() runs the next step.  New gradients are
        copied into the tensors the tables point to before each replay."""
        if self.cfg.scale_mode == capi.SCALE_POWER and self.v0 is None:
            raise ValueError("set the start vectors before capturing")
        self.reserve()
        torch.cuda.synchronize()
        graphs = {}
        for refresh in ((True,) if self.cfg.update_every == 1 else (True, False)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._enqueue(g_table, u_table, refresh)
            graphs[refresh] = g
        torch.cuda.synchronize()
        return StepGraph(self, graphs, (g_table, u_table))

    def update_roots(self, stream=None):
        c = self.cfg
        scale_power(self.factors, c.eps_rel, c.scale_mode, self.v0, c.pi_steps, c.safety, self.scale,
                    self.status, self.ws["scale"], stream)
        if c.solver == "newton":
            invroot_newton(self.factors, self.scale, c.p, c.variant, c.iters, self.roots, self.status,
                           self.resid, self.ws["root"], stream)
        else:
            invroot_cheby(self.factors, self.scale, c.p, c.degree, c.interval_eps, c.prec, self.roots,
                          self.status, self.ws["root"], stream)


class StepGraph:
    """Captured optimizer steps of a ShampooBlocks: replay() enqueues the next
    step (refresh or cached roots, as the state's step count says) as one graph
    launch on the current stream and advances the step count."""

    def __init__(self, state, graphs, tables):
        self.state = state
        self.graphs = graphs
        self._tables = tables  # keep the descriptor tables alive

    def replay(self):
        self.graphs[self.state.refresh_due].replay()
        self.state.t += 1
