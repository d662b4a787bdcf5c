"""The oracle's own prefix trie over valid catalog SIDs. Test infrastructure only.

flashrec 0.1.0, Features > Decoding ("SID constraint"): decoding is restricted to
a catalog of valid semantic IDs through a (dense or CSR-sparse) trie; SPRINT
summary, inference paragraph: only valid SIDs in a prefix trie are scored.

Construction (plain definition, not a data structure to be fast):
  * a SID (c_0, ..., c_{L-1}) is packed big-endian into one integer;
  * P_d = sorted distinct depth-d prefixes (key >> 8(L-d)); P_0 = {empty prefix};
  * node id of prefix p at depth d = off_d + rank of p in P_d, with
    off_d = |P_0| + ... + |P_{d-1}| (depth-major, lexicographic numbering);
  * children(p) = the ascending codes c with p.c in P_{d+1};
  * leaf_item(p) = the lowest catalog row whose SID is p (the catalog maps SIDs to
    items many-to-one, flashrec 0.1.0 Quickstart's sid2pid catalog file; the
    reading taken: duplicates collapse onto the lowest row).
"""
from __future__ import annotations

import numpy as np


class OracleTrie:
    def __init__(self, sids, V: int = 256):
        sids = np.asarray(sids)
        if sids.ndim != 2 or sids.shape[0] == 0:
            raise ValueError("sids must be a non-empty [n_items, L] array")
        if sids.min() < 0 or sids.max() >= V:
            raise ValueError("code out of range")
        self.V = int(V)
        self.L = int(sids.shape[1])
        keys = np.zeros(sids.shape[0], dtype=np.uint64)
        for j in range(self.L):
            keys = keys * np.uint64(256) + sids[:, j].astype(np.uint64)
        # np.unique returns the first (lowest) row index of each distinct key
        self.leaf_keys, self.leaf_item = np.unique(keys, return_index=True)
        self.leaf_item = self.leaf_item.astype(np.int64)
        self.P = []
        for d in range(self.L + 1):
            shift = np.uint64(8 * (self.L - d))
            self.P.append(np.unique(self.leaf_keys >> shift) if d > 0
                          else np.zeros(1, dtype=np.uint64))
        self.off = [0]
        for d in range(self.L + 1):
            self.off.append(self.off[-1] + len(self.P[d]))

    # ------------------------------------------------------------------ queries
    @property
    def n_distinct(self) -> int:
        return len(self.leaf_keys)

    @property
    def nodes_per_depth(self):
        return [len(p) for p in self.P]

    def node_id(self, depth: int, prefix) -> int:
        prefix = np.uint64(prefix)
        rank = int(np.searchsorted(self.P[depth], prefix))
        if rank >= len(self.P[depth]) or self.P[depth][rank] != prefix:
            raise KeyError(f"prefix {int(prefix):#x} not in catalog at depth {depth}")
        return self.off[depth] + rank

    def prefix_of(self, node: int):
        """(depth, packed prefix) of a node id."""
        d = int(np.searchsorted(np.asarray(self.off), node, side="right")) - 1
        return d, int(self.P[d][node - self.off[d]])

    def children(self, depth: int, prefix):
        """Ascending child codes of ``prefix`` (a depth-``depth`` node) and their node ids."""
        nxt = self.P[depth + 1]
        base = np.uint64(prefix) * np.uint64(256)
        lo = int(np.searchsorted(nxt, base, side="left"))
        hi = int(np.searchsorted(nxt, base + np.uint64(255), side="right"))
        codes = (nxt[lo:hi] & np.uint64(255)).astype(np.int64)
        nodes = self.off[depth + 1] + np.arange(lo, hi, dtype=np.int64)
        return codes, nodes

    def contains(self, sid_packed) -> bool:
        k = np.uint64(sid_packed)
        i = int(np.searchsorted(self.leaf_keys, k))
        return i < len(self.leaf_keys) and self.leaf_keys[i] == k

    def item_of(self, sid_packed) -> int:
        k = np.uint64(sid_packed)
        i = int(np.searchsorted(self.leaf_keys, k))
        if i >= len(self.leaf_keys) or self.leaf_keys[i] != k:
            raise KeyError("not a catalog SID")
        return int(self.leaf_item[i])

    def unpack(self, sid_packed, depth=None):
        depth = self.L if depth is None else depth
        k = int(sid_packed)
        return tuple((k >> (8 * (depth - 1 - j))) & 255 for j in range(depth))
