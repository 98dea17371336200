"""Sketch Attention (FlashSA-style) forward and backward for MI355X (gfx950).

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``csrc/``, declared in ``include/sa.h`` at the repository root).  The
``sa`` module is a thin ctypes binding with the same entry-point names; it
loads the library on first use and raises if it has not been built.
``synth`` draws seeded synthetic inputs and holds none of the method's
arithmetic.
"""

__all__ = ["sa", "synth"]
