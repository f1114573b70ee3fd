"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and the oracle.

This module only draws random numbers and lays out shapes; it holds none of
the preconditioner's arithmetic.  Every array is drawn in float64 with
numpy's PCG64 seeded by a SeedSequence key (config id, tag, indices) and
rounded once to float32; those float32 bytes are what both sides consume.

Workloads (the pages train a ~1B Llama-style model on C4, which is not
available here; gradients are Gaussian stand-ins of the same shapes):
  config 1  8 SPD blocks 64x64: A_i = G_i G_i^T / 128 + 1e-6 I, G_i ~ N(0,1)
            of shape 64x128, numpy seed 0.
  config 2  one 1024x1024 linear-layer gradient per step, N(0, 0.02^2),
            5 steps, blocked 4x4 at B = 256.
  config 3  360M-shaped transformer: 24 layers, hidden 1024, MLP 4096
            (Wq, Wk, Wv, Wo 1024x1024; W_up 4096x1024; W_down 1024x4096),
            N(0, 0.02^2) gradients, B = 1024 -> 288 blocks.
  config 4  64 SPD blocks 512x512, A = Q diag(lambda) Q^T, Q Haar-random
            orthogonal, lambda log-uniform in [1e-8, 1].
  config 5  1.3B-shaped transformer: 24 layers, hidden 2048, MLP 8192,
            B = 2048 -> 288 blocks.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass

import numpy as np

TAG_G = 1        # gradients
TAG_Q = 2        # Haar orthogonal factors
TAG_LAM = 3      # eigenvalues
TAG_V0 = 4       # power-iteration start vectors
TAG_SUBSET = 5   # which blocks a sampled parity check looks at
TAG_SPD = 6      # generic SPD test blocks
TAG_EDGE = 7     # generic gradient-like test blocks

GRAD_STD = 0.02


def rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def _threads():
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


# ---------------------------------------------------------------------------
# Power-iteration start vectors
# ---------------------------------------------------------------------------

def start_vectors(cfg, nfactors, B, r=32, first=0):
    """[nfactors, B, r] float32 N(0,1) start vectors, factor i seeded (cfg, TAG_V0, i)."""
    out = np.empty((nfactors, B, r), dtype=np.float32)
    for j in range(nfactors):
        out[j] = rng(cfg, TAG_V0, first + j).standard_normal((B, r)).astype(np.float32)
    return out


def start_vector(cfg, index, B, r=32):
    return rng(cfg, TAG_V0, index).standard_normal((B, r)).astype(np.float32)


# ---------------------------------------------------------------------------
# Config 1 and config 4: SPD factors given directly
# ---------------------------------------------------------------------------

def config1_factors():
    g = np.random.Generator(np.random.PCG64(0)).standard_normal((8, 64, 128))
    a = np.einsum("bik,bjk->bij", g, g) / 128.0 + 1e-6 * np.eye(64)
    return a.astype(np.float32)


def haar_orthogonal(gen, n):
    """Haar-random orthogonal matrix: QR of a Gaussian with the signs of
    diag(R) moved into Q (Mezzadri 2007)."""
    z = gen.standard_normal((n, n))
    q, r = np.linalg.qr(z)
    return q * np.sign(np.diag(r))


def config4_factor(i, B=512, lo=-8.0, hi=0.0):
    """(A fp32, Q float64, lambda float64) for block i of config 4."""
    q = haar_orthogonal(rng(4, TAG_Q, i), B)
    lam = 10.0 ** rng(4, TAG_LAM, i).uniform(lo, hi, B)
    a = (q * lam) @ q.T
    a = 0.5 * (a + a.T)
    return a.astype(np.float32), q, lam


def config4_factors(n=64, B=512):
    return np.stack([config4_factor(i, B)[0] for i in range(n)])


def spd_factors(key, n, B, cond=1e3):
    """Generic SPD test factors with eigenvalues log-uniform in [1/cond, 1]."""
    out = np.empty((n, B, B), dtype=np.float32)
    for i in range(n):
        q = haar_orthogonal(rng(TAG_SPD, key, i, 0), B)
        lam = 10.0 ** rng(TAG_SPD, key, i, 1).uniform(-np.log10(cond), 0.0, B)
        a = (q * lam) @ q.T
        out[i] = (0.5 * (a + a.T)).astype(np.float32)
    return out


# ---------------------------------------------------------------------------
# Gradients: single matrices and model-shaped sets of layer weights
# ---------------------------------------------------------------------------

def gaussian(key, shape, std=GRAD_STD):
    return (rng(*key).standard_normal(shape) * std).astype(np.float32)


def config2_gradient(step):
    """1024x1024 N(0, 0.02^2) gradient of config 2 at step t (t = 1..5)."""
    return gaussian((2, TAG_G, step), (1024, 1024))


@dataclass(frozen=True)
class ModelSpec:
    """2D weights of a Llama-style stack, in PyTorch [out, in] layout."""
    layers: int
    hidden: int
    mlp: int

    def weights(self):
        h, m = self.hidden, self.mlp
        shapes = [("Wq", (h, h)), ("Wk", (h, h)), ("Wv", (h, h)), ("Wo", (h, h)),
                  ("W_up", (m, h)), ("W_down", (h, m))]
        return [(layer, k, name, shape) for layer in range(self.layers)
                for k, (name, shape) in enumerate(shapes)]


MODEL_360M = ModelSpec(24, 1024, 4096)
MODEL_1_3B = ModelSpec(24, 2048, 8192)


@dataclass(frozen=True)
class BlockRef:
    weight: int      # index into ModelSpec.weights()
    row0: int
    col0: int
    rows: int
    cols: int


def block_layout(shapes, B):
    """Split each weight of `shapes` (list of (rows, cols)) into B x B blocks,
    row-major within a weight, weights in order; edge blocks may be partial."""
    out = []
    for w, (m, n) in enumerate(shapes):
        for r0 in range(0, m, B):
            for c0 in range(0, n, B):
                out.append(BlockRef(w, r0, c0, min(B, m - r0), min(B, n - c0)))
    return out


def model_gradient(cfg, layer, mat, shape):
    return gaussian((cfg, TAG_G, layer, mat), shape)


def model_gradients(cfg, spec, threads=None):
    """All layer gradients of a ModelSpec, drawn in parallel (one seed per weight)."""
    ws = spec.weights()
    with _cf.ThreadPoolExecutor(threads or _threads()) as ex:
        return list(ex.map(lambda w: model_gradient(cfg, w[0], w[1], w[3]), ws))


def sampled_blocks(cfg, nblocks, count=2, fixed=(0, 1)):
    """Block indices a sampled parity check covers: the fixed ones (first,
    second, last) plus `count` drawn with seed (cfg, TAG_SUBSET)."""
    picks = set(i for i in fixed if i < nblocks)
    picks.add(nblocks - 1)
    extra = rng(cfg, TAG_SUBSET).choice(nblocks, size=min(count, nblocks), replace=False)
    picks.update(int(i) for i in extra)
    return sorted(picks)


def ragged_gradients(key, shapes, std=1.0):
    """Gradient-like matrices of arbitrary shapes (edge-case tests)."""
    return [(rng(TAG_EDGE, key, i).standard_normal(s) * std).astype(np.float32)
            for i, s in enumerate(shapes)]
