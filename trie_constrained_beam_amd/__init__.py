"""Catalog-constrained wide-beam expansion on MI355X (gfx950).

The beam step and single-pass catalog scoring run in libtcb.so (hand-written HIP
kernels behind the C ABI of include/tcb.h); this package is its Python binding
(``Trie``, ``Beams``, ``score_catalog``) plus the seeded workload generators in ``synth``.
"""
from . import _lib
from .api import Beams, Trie, invalid_rate, score_catalog, score_workspace_bytes
from ._lib import TcbError
from .wave import run_wave

__all__ = ["Beams", "Trie", "TcbError", "run_wave", "invalid_rate", "score_catalog", "score_workspace_bytes"]
