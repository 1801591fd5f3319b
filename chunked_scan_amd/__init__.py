"""chunked_scan_amd -- chunked causal linear attention with a segmented state scan on MI355X.

The compute lives in a C-ABI shared library of hand-written HIP kernels for gfx950
(``liblachunk.so``, declared in ``include/la_chunk.h``).  This package holds the thin ctypes
binding to it and the seeded synthetic input generators.  Importing the package does not load
the library; the first call of a binding function does, and fails loudly if it is missing.
"""
__all__ = ["la_chunk_fwd", "la_state_scan", "la_state_correct", "la_cumdecay", "inputs"]


def __getattr__(name):
    if name in ("la_chunk_fwd", "la_state_scan", "la_state_correct", "la_cumdecay",
                "la_chunk_fwd_nodes", "lib", "LaError", "Shape"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
