"""KronQ per-layer post-training quantization solver for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library libkq.so (include/kq.h, HIP kernels under csrc/);
this package only binds it (``_lib``) and orders the calls for one layer (``layer``).
"""
from . import _lib  # noqa: F401

__all__ = ["_lib"]
