"""Fused, deterministic mixture-of-experts layer for AMD MI355X (gfx950).

The compute path is libmok.so (HIP kernels behind the C ABI in include/mok.h);
`mok` is its ctypes binding and `layer` the torch buffer plumbing.  Importing
the package does not load the library; the first call does, and fails loudly
if it has not been built.
"""
from . import mok  # noqa: F401

__all__ = ["mok", "layer", "build"]
