"""Routed MoE over a shared expert slot cache, native on MI355X (gfx950).

The compute path lives in libscr.so (HIP kernels behind a C ABI, declared in
include/scr.h); ``_lib`` binds it with ctypes and ``layer`` drives it with
PyTorch-owned memory and streams.  Importing the package does not touch the
GPU; the first call into the library loads libscr.so and raises ImportError
if it has not been built.
"""
from . import _lib  # noqa: F401

__all__ = ["_lib"]
