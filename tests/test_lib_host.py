"""libtcb.so on the host (no GPU): exported symbols, trie builder, argument errors.

The builder's numbering is checked against the oracle's independent trie: both
number nodes depth-major and lexicographically (a contract stated in include/tcb.h)
but share no code.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
from trie_constrained_beam_amd import Trie, TcbError, _lib, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            names |= set(re.findall(r"^\s*(?:tcb_status|void|const char \*)\s*\*?\s*(tcb_\w+)\s*\(",
                                    text, flags=re.M))
    return names


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 19
    h = C.CDLL(_lib.LIB_PATH)
    missing = [n for n in sorted(names) if not hasattr(h, n)]
    assert not missing, missing
    assert names == set(_lib.SIGNATURES), names ^ set(_lib.SIGNATURES)
    assert _lib.lib().tcb_version().decode().startswith("tcb")


@pytest.mark.parametrize("V,L,n,mask_depths,seed", [
    (256, 3, 5000, 3, 0), (256, 4, 3000, 0, 1), (5, 3, 80, 2, 2), (2, 1, 2, 1, 3),
    (256, 5, 4000, 5, 4), (17, 2, 200, 1, 5)])
def test_builder_matches_oracle_numbering(V, L, n, mask_depths, seed):
    rng = np.random.default_rng(seed)
    hi = min(V, 12) if L >= 3 else V
    cat = rng.integers(0, hi, size=(n, L)).astype(np.uint8)
    t = Trie(cat, V=V, mask_depths=mask_depths)
    o = oracle.OracleTrie(cat.astype(np.int64), V=V)
    assert t.nodes_per_depth == o.nodes_per_depth
    assert t.n_distinct == o.n_distinct
    assert t.node_offset[:-1] == o.off[:-1]
    cb, cc, li = t.host_arrays()
    for d in range(L):
        for i, p in enumerate(o.P[d]):
            node = o.off[d] + i
            codes, nodes = o.children(d, int(p))
            assert list(range(cb[node], cb[node + 1])) == list(nodes)
            assert list(cc[cb[node]:cb[node + 1]]) == list(codes)
    assert np.array_equal(li, o.leaf_item)


def test_builder_dedupes_to_lowest_row():
    cat = np.array([[3, 1], [0, 2], [3, 1], [0, 2], [1, 1]], dtype=np.uint8)
    t = Trie(cat, V=4)
    assert t.n_distinct == 3
    _, _, li = t.host_arrays()
    assert list(li) == [1, 4, 0]          # leaves in order (0,2), (1,1), (3,1)


def test_builder_synthetic_catalog_scale():
    cat = synth.catalog(200_000, 4, ("zipf",) * 4, [21, 1])
    t = Trie(cat)
    o = oracle.OracleTrie(cat)
    assert t.nodes_per_depth == o.nodes_per_depth


def _err(fn, *args):
    code = fn(*args)
    return code


def test_build_errors():
    lib = _lib.lib()
    out = C.c_void_p()
    cat = np.zeros((4, 3), dtype=np.uint8)
    cat[2, 1] = 9
    assert lib.tcb_build_trie(None, 4, 3, 256, 0, C.byref(out)) == -1
    assert lib.tcb_build_trie(cat.ctypes.data, 0, 3, 256, 0, C.byref(out)) == -1
    assert lib.tcb_build_trie(cat.ctypes.data, 4, 9, 256, 0, C.byref(out)) == -2
    assert lib.tcb_build_trie(cat.ctypes.data, 4, 3, 1, 0, C.byref(out)) == -2
    assert lib.tcb_build_trie(cat.ctypes.data, 4, 3, 257, 0, C.byref(out)) == -2
    assert lib.tcb_build_trie(cat.ctypes.data, 4, 3, 8, 0, C.byref(out)) == -2     # code 9 >= V
    assert b"code 9" in lib.tcb_last_error()
    assert lib.tcb_build_trie(cat.ctypes.data, 4, 3, 256, 4, C.byref(out)) == -1  # mask_depths > L
    with pytest.raises(TcbError):
        Trie(cat, V=8)


def test_wave_errors_before_device_work():
    lib = _lib.lib()
    cat = synth.catalog(1000, 3, ("uniform",) * 3, [22, 1])
    t = Trie(cat)
    nb = C.c_size_t()
    assert lib.tcb_beams_workspace_bytes(t.handle, 0, 4, 8, C.byref(nb)) == -1
    assert lib.tcb_beams_workspace_bytes(t.handle, 64, 4, 5000, C.byref(nb)) == -1
    assert lib.tcb_beams_workspace_bytes(t.handle, 64, 4, 8, C.byref(nb)) == 0 and nb.value > 0
    out = C.c_void_p()
    fake = C.c_void_p(1 << 20)           # never dereferenced: validation fails first
    # trie not uploaded
    assert lib.tcb_beams_create(t.handle, 64, 4, 8, 0, fake, nb.value, None, C.byref(out)) == -4
    # upload checks run before any copy
    assert lib.tcb_trie_upload(t.handle, fake, 16, None) == -5
    assert lib.tcb_trie_upload(t.handle, C.c_void_p((1 << 20) + 8), 1 << 30, None) == -5
    assert lib.tcb_beam_step(None, fake, 256, 0, None) == -1


@pytest.mark.parametrize("L,per", [(1, 4), (4, 4), (5, 8), (8, 8)])
def test_score_host_sizes(L, per):
    """Leaf codes take 4 bytes per distinct SID up to L = 4 and 8 above; the scoring
    workspace grows with the number of users (one table and maxima set per user group)."""
    cat = synth.catalog(200 if L == 1 else 3000, L, ("uniform",) * L, [90, L])
    t = Trie(cat)
    nb = C.c_size_t()
    _lib.check(_lib.lib().tcb_trie_codes_bytes(t.handle, C.byref(nb)))
    assert nb.value == t.n_distinct * per
    sizes = []
    for users in (1, 16, 32, 33, 200):
        _lib.check(_lib.lib().tcb_score_workspace_bytes(t.handle, users, C.byref(nb)))
        assert nb.value % 256 == 0
        sizes.append(nb.value)
    assert sizes == sorted(sizes) and sizes[-1] > sizes[0]
    with pytest.raises(TcbError, match="ARG"):
        _lib.check(_lib.lib().tcb_score_workspace_bytes(t.handle, 0, C.byref(nb)))


def test_score_requires_uploaded_trie():
    cat = synth.catalog(500, 3, ("uniform",) * 3, [91, 1])
    t = Trie(cat)
    with pytest.raises(TcbError, match="STATE"):
        _lib.check(_lib.lib().tcb_score_catalog(t.handle, 1, C.c_void_p(16), 0, None, None, 0, 1.0, 4,
                                                C.c_void_p(16), None, C.c_void_p(16), None,
                                                C.c_void_p(256), 1 << 20, None))
