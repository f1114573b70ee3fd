"""Helpers shared by the GPU parity tests: run stages of the HIP path through
the C ABI on seeded inputs and compare with the float64 oracle."""
import json
import os

import numpy as np
import torch

from oracle import shampoo_oracle as O
from inverse_root_preconditioning_amd import capi
from inverse_root_preconditioning_amd import pipeline as PL

TOL_F32 = 1e-4    # relative Frobenius per factor, fp32 paths
TOL_BF16 = 2e-2   # relative Frobenius per factor, bf16-input paths

_REPORT = os.environ.get("SHAMPOO_PARITY_REPORT")


def report(name, **vals):
    """Append measured errors to a JSON-lines report when one is requested."""
    line = {"case": name}
    line.update({k: (float(v) if isinstance(v, (np.floating, float, int, np.integer)) else v) for k, v in vals.items()})
    print(json.dumps(line), flush=True)
    if _REPORT:
        with open(_REPORT, "a") as f:
            f.write(json.dumps(line) + "\n")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def max_rel(xs, refs):
    return max(O.relative_frobenius(x, r) for x, r in zip(xs, refs))


def gpu_scale(F, eps_rel, mode, V0=None, steps=20, safety=2.0):
    """F: [nf, B, B] fp32 device tensor.  Returns (scale, status) device tensors."""
    nf = F.shape[0]
    sc, st = PL.new_scale(nf, F.device)
    PL.scale_power(F, eps_rel, mode, V0, steps, safety, sc, st)
    return sc, st


def gpu_roots(F, sc, st, method, iters=10, p=4, variant=capi.NDB, degree=24, delta=1e-12, prec=capi.F32,
              resid=False):
    X = torch.empty_like(F)
    R = None
    if method == "newton":
        if resid:
            passes = 1 if (p == 2 or (variant & 0xff) in (capi.CN, capi.CN_F16)) else 2
            R = torch.full((F.shape[0], passes * iters), -1.0, dtype=torch.float32, device=F.device)
        PL.invroot_newton(F, sc, p, variant, iters, X, st, R)
    else:
        PL.invroot_cheby(F, sc, p, degree, delta, prec, X, st)
    return X, R


VARIANT_NAME = {capi.NDB: "ndb", capi.NDB_Z: "ndb", capi.CN: "cn", capi.CN_F16: "cn"}
CHAINING = {capi.NDB: "Y", capi.NDB_Z: "Z", capi.CN: "Y", capi.CN_F16: "Y"}


def oracle_scale(F, eps_rel, mode, V0, steps=20, safety=2.0):
    return O.scale_factor(F, eps_rel, "power" if mode == capi.SCALE_POWER else "frobenius", V0, steps, safety)


def oracle_root(F, sc, method, iters=10, p=4, variant=capi.NDB, degree=24, delta=1e-12):
    if method == "newton":
        return O.invroot(F, sc, VARIANT_NAME[variant], iters=iters, p=p, chaining=CHAINING[variant])
    return O.invroot(F, sc, "cheby", p=p, degree=degree, delta=delta)


def fill_factor(B, per_factor_tiles, base, cus=256, rounds=4):
    """How many copies of `base` checked factors a stack needs so that a launch
    over it has at least `rounds` x `cus` workgroups of `per_factor_tiles`
    tiles per factor.  The library takes the 256 x 256 tiles only when their
    grid fills the GPU in whole rounds or in at least four rounds (else smaller
    tiles), so tests meant for the large-tile kernels replicate their factors."""
    need = -(-(rounds * cus) // per_factor_tiles)
    return -(-need // base)


def upper_tiles(B, T):
    t = B // T
    return t * (t + 1) // 2
