"""int4 routed-expert MoE block for MI355X (gfx950): HIP kernels behind a C ABI.

The native library (libmoe_amd.so, built by ``build.py``) holds every step of
the path; ``api`` is a thin ctypes binding that marshals torch tensors.
"""
from ._lib import MoeError, lib  # noqa: F401
