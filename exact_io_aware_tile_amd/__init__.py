"""MI355X (gfx950) exact attention: tiled online-softmax kernels behind a C ABI.

``exact_io_aware_tile_amd.fa`` is the thin binding over ``libfa_gfx950.so``
(see ``include/fa.h``); ``exact_io_aware_tile_amd.inputs`` holds the seeded
synthetic input generators.  Importing the package loads nothing; the HIP
library is loaded on first use and its absence is an error.
"""
__all__ = ["fa", "inputs"]
