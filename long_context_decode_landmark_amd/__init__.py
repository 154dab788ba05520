"""MI355X (gfx950) implementation of LowRAM's decode-time selective-reconstruction attention.

The decode step runs in the hand-written HIP kernels of ``liblowram.so``
(C ABI in include/lowram.h); ``native`` is its thin ctypes binding.  Build the
library in-tree with ``long_context_decode_landmark_amd.build.build()``.
"""
from . import native  # noqa: F401
from .native import LowramError  # noqa: F401

__all__ = ["native", "LowramError"]
