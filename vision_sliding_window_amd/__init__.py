"""Fused 2D Neighborhood Attention forward for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libna2d.so`` built from ``csrc/``; the
Python binding in ``na2d.py`` only marshals arguments to its C ABI
(``include/na2d.h``).  ``inputs.py`` draws seeded synthetic inputs.
"""
__all__ = ["na2d", "inputs"]
