"""Catalog-constrained wide-beam expansion on MI355X (gfx950).

The beam step runs in libtcb.so (hand-written HIP kernels behind the C ABI of
include/tcb.h); this package is its Python binding (``Trie``, ``Beams``) plus the
seeded workload generators in ``synth``.
"""
from . import _lib
from .api import Beams, Trie, invalid_rate
from ._lib import TcbError
from .wave import run_wave

__all__ = ["Beams", "Trie", "TcbError", "run_wave", "invalid_rate"]
