"""Build the HIP library in-tree: lib/libshampoo_mi355x.so for gfx950.

    python -m inverse_root_preconditioning_amd.build

hipcc cross-compiles without a GPU.  Packed fp32 instructions are disabled
for all device code (`-packed-fp32-ops`); the host pass warns that it does
not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libshampoo_mi355x.so")
ARCH = os.environ.get("SHAMPOO_OFFLOAD_ARCH", "gfx950")

SOURCES = ["shampoo.hip"]
HEADERS = ["common.h", "gemm_f32.h", "gemm_bf16.h", "kernels_misc.h"]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def command(out=LIB):
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"),
            "-o", out] + [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose=False):
    """Compile the library (always recompiles).  Raises on failure."""
    os.makedirs(LIBDIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
