"""Sparse Mixture-of-Experts feed-forward layer for MI355X (gfx950).

route -> permute -> grouped SwiGLU GEMMs -> combine, as hand-written HIP
kernels behind a C ABI (``include/moe_mi355x.h``).  ``moe`` holds the thin
torch-facing binding; ``inputs`` holds the seeded synthetic input generator.
The HIP library is loaded lazily on first use and its absence is an error.
"""
import importlib

__all__ = ["moe", "inputs"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
