"""Exact quantile balancing (EQB) and K3 uniform-bin bias updates for an
auxiliary-loss-free MoE router, on MI355X (gfx950).

The computation lives in libqb.so (HIP kernels behind the C ABI of
include/qb.h); ``qb`` is its Python binding and ``synth`` the seeded input
generators.  Importing the package loads nothing; ``qb.lib()`` loads the
library on first use.
"""
__all__ = ["qb", "synth"]
__version__ = "0.1.0"
