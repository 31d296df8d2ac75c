"""Semantic-ID beam-search decode step for AMD Instinct MI355X (gfx950).

The compute runs in libgr_beam.so (hand-written HIP kernels + C ABI declared
in include/gr_beam.h); ``_lib`` binds it with ctypes under the same names and
``BeamEngine`` keeps the torch-owned device buffers.  Importing this package
does not load the library; the first call does, and fails loudly if it was
not built.
"""
from . import _lib  # noqa: F401
from ._lib import GrError, lib  # noqa: F401
from .engine import BeamEngine, Scheduler, to_device  # noqa: F401
