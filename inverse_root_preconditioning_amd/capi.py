"""ctypes binding of the C ABI declared in include/shampoo.h.

Argument marshalling only: every function here forwards to the entry point of
the same name in lib/libshampoo_mi355x.so; pointers are passed as integers
(device addresses, e.g. ``tensor.data_ptr()``) and the stream as its raw
handle (``torch.cuda.current_stream().cuda_stream``).  The library is loaded
on first use; if it has not been built the call raises -- there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libshampoo_mi355x.so")

# Return codes
OK = 0
EINVAL = -1
EUNSUPPORTED = -2
EWORKSPACE = -3
EHIP = -4
ESCRATCH = -5
NOALLOC_SCRATCH_BYTES = 1 << 20
# Per-factor status bits
BLK_NONFINITE = 1
BLK_ZERO = 2
BLK_NONPOS_RQ = 4
BLK_RESID_GROWTH = 8
# Precision
F32 = 0
BF16_IN = 1
# Scaling modes
SCALE_POWER = 0
SCALE_FROBENIUS = 1
# Newton variants
NDB = 0
NDB_Z = 1
CN = 2
CN_F16 = 3
# Modifier bit for variant (newton) / prec (cheby): compute symmetric products in full
FULL_PRODUCTS = 0x100
SYM_COUPLING = 0x200      # opt-in: coupling products from upper tiles (faster, less stable)
# Workspace op ids
OP_ACCUMULATE = 1
OP_SCALE = 2
OP_NEWTON = 3
OP_CHEBY = 4
OP_PRECONDITION = 5
OP_GRAFT = 6

ABI_VERSION = 2


class shampoo_block(ctypes.Structure):
    _fields_ = [("ptr", c_void_p), ("ld", c_int64), ("rows", c_int32), ("cols", c_int32)]


class shampoo_scale(ctypes.Structure):
    _fields_ = [("c", c_float), ("eps", c_float), ("lambda_", c_float), ("trace", c_float)]


class ShampooError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


# Timing-hook kernel families
TIME_OFF = 0
TIME_NDB_PAIR = 1
TIME_NDB_P = 2
TIME_CLENSHAW = 4
TIME_CN_M = 8
TIME_ALL = 15

_SIGNATURES = {
    "shampoo_abi_version": (c_int, []),
    "shampoo_timing_hook": (c_int, [c_int, c_void_p, c_void_p, c_int]),
    "shampoo_timing_count": (c_int, []),
    "shampoo_strerror": (ctypes.c_char_p, [c_int]),
    "shampoo_workspace_bytes": (c_size_t, [c_int, c_int64, c_int, c_int, c_int]),
    "shampoo_accumulate": (c_int, [c_void_p, c_int64, c_int, c_void_p, c_float, c_float, c_int,
                                   c_void_p, c_size_t, c_void_p]),
    "shampoo_scale_power": (c_int, [c_void_p, c_int64, c_int, c_float, c_int, c_void_p, c_int, c_int,
                                    c_float, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "shampoo_invroot_newton": (c_int, [c_void_p, c_void_p, c_int64, c_int, c_int, c_int, c_int,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "shampoo_invroot_cheby": (c_int, [c_void_p, c_void_p, c_int64, c_int, c_int, c_int, c_double, c_int,
                                      c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "shampoo_precondition": (c_int, [c_void_p, c_void_p, c_int64, c_int, c_void_p, c_int,
                                     c_void_p, c_size_t, c_void_p]),
    "shampoo_graft_update": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int,
                                     c_float, c_float, c_float, c_float, c_int, c_void_p,
                                     c_void_p, c_size_t, c_void_p]),
    "shampoo_graft_update_noalloc": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int,
                                             c_float, c_float, c_float, c_float, c_int, c_void_p, c_void_p]),
}

EXPORTED = tuple(_SIGNATURES)

_lib = None


def load(path=None):
    """Load (once) and return the library; raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"HIP library not built: {p} is missing "
                           "(run `python -m inverse_root_preconditioning_amd.build`)")
    # PyTorch ships its own HIP runtime.  It is loaded first so that this
    # library binds to that copy: with a second runtime in the process, the
    # launches here would not see the streams and memory the caller got from
    # PyTorch and would fail.
    import torch  # noqa: F401
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.shampoo_abi_version() != ABI_VERSION:
        raise RuntimeError("libshampoo_mi355x.so ABI version mismatch")
    if path is None:
        _lib = lib
    return lib


def strerror(code):
    return load().shampoo_strerror(code).decode()


def check(code, where="shampoo"):
    if code != OK:
        raise ShampooError(code, where)
    return code


def shampoo_abi_version():
    return load().shampoo_abi_version()


def shampoo_strerror(code):
    return strerror(code)


def shampoo_workspace_bytes(op, count, B, variant_or_degree, prec):
    return load().shampoo_workspace_bytes(op, count, B, variant_or_degree, prec)


def shampoo_accumulate(g_blocks, nblocks, B, factors, alpha, gamma, prec, ws, ws_bytes, stream):
    return load().shampoo_accumulate(g_blocks, nblocks, B, factors, alpha, gamma, prec, ws, ws_bytes, stream)


def shampoo_scale_power(factors, nfactors, B, eps_rel, mode, v0, r, steps, safety, scale_out, status,
                        ws, ws_bytes, stream):
    return load().shampoo_scale_power(factors, nfactors, B, eps_rel, mode, v0, r, steps, safety,
                                      scale_out, status, ws, ws_bytes, stream)


def shampoo_invroot_newton(factors, scale, nfactors, B, p, variant, iters, x_out, resid_out, status,
                           ws, ws_bytes, stream):
    return load().shampoo_invroot_newton(factors, scale, nfactors, B, p, variant, iters, x_out, resid_out,
                                         status, ws, ws_bytes, stream)


def shampoo_invroot_cheby(factors, scale, nfactors, B, p, degree, interval_eps, prec, x_out, status,
                          ws, ws_bytes, stream):
    return load().shampoo_invroot_cheby(factors, scale, nfactors, B, p, degree, interval_eps, prec, x_out,
                                        status, ws, ws_bytes, stream)


def shampoo_precondition(x_roots, g_blocks, nblocks, B, u_blocks, prec, ws, ws_bytes, stream):
    return load().shampoo_precondition(x_roots, g_blocks, nblocks, B, u_blocks, prec, ws, ws_bytes, stream)


def shampoo_timing_hook(families, events, fam_out, capacity):
    return load().shampoo_timing_hook(families, events, fam_out, capacity)


def shampoo_timing_count():
    return load().shampoo_timing_count()


def shampoo_graft_update(g_blocks, u_blocks, param_blocks, m_blocks, v_blocks, nblocks, B, lr, beta1, beta2,
                         eps, step, scale_out, ws, ws_bytes, stream):
    return load().shampoo_graft_update(g_blocks, u_blocks, param_blocks, m_blocks, v_blocks, nblocks, B, lr,
                                       beta1, beta2, eps, step, scale_out, ws, ws_bytes, stream)


def shampoo_graft_update_noalloc(g_blocks, u_blocks, param_blocks, m_blocks, v_blocks, nblocks, B, lr, beta1,
                                 beta2, eps, step, scale_out, stream):
    return load().shampoo_graft_update_noalloc(g_blocks, u_blocks, param_blocks, m_blocks, v_blocks, nblocks, B,
                                               lr, beta1, beta2, eps, step, scale_out, stream)
