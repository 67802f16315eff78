"""Quantised Mixture-of-Experts layer (sigmoid top-k router, int4 x int8 SwiGLU
experts, MXFP4 variant, HBM expert cache) for AMD MI355X / gfx950.

The compute runs in libmoe.so (hand-written HIP kernels behind the C ABI of
include/moe.h).  ``abi`` is the ctypes binding with the C names, ``layer`` a
helper that keeps one layer resident on the GPU, ``synth`` the seeded input
generators.  Importing the package does not load the library; the first call
does, and fails if it has not been built.
"""
from . import abi, synth  # noqa: F401

__all__ = ["abi", "synth"]
