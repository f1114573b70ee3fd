"""MI355X-native Shampoo block-preconditioner hot path.

The compute path lives in the HIP library built from ``csrc/`` (C ABI declared
in ``include/shampoo.h``); ``capi`` is its ctypes binding and ``pipeline`` the
torch-tensor convenience layer.  ``workloads`` holds the seeded synthetic
inputs.  Importing the package does not load the library; the first call
into ``capi`` does, and raises if it has not been built.
"""
__all__ = ["capi", "pipeline", "workloads"]
