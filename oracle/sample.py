"""Gumbel top-k without replacement over beams, written plainly in float64.
Test infrastructure only.

Above temperature 0 the serving API returns the beams of a Gumbel top-k without
replacement (flashrec 0.1.0, Features > Serving, "API"). The pages give no more
than that; the readings taken here (each also listed in the design doc):

  * temperature tempers every step's distribution: a row's children are scored
    with the masked log-softmax of x / T (the same normaliser choice as at T = 0),
    and a beam's log-probability phi is the sum of those tempered terms;
  * "without replacement" is meant over whole SIDs: the request's beams are an
    exact sample of n distinct SIDs without replacement from the tempered sequence
    model (Plackett-Luce / Gumbel-top-k over complete SIDs). The plain way to get
    that from a level-by-level beam is stochastic beam search (Kool, van Hoof and
    Welling, ICML 2019): every beam carries phi and a perturbed key G (the root
    has phi = 0, G = 0); a child c of beam r draws g_c = phi_c + Gumbel(0, 1) and
    gets the key of the top-down sample conditioned on its siblings' maximum being
    the parent's key,
        G_c = -log(exp(-G_r) - exp(-Z_r) + exp(-g_c)),   Z_r = max over siblings g,
    and the request keeps its n best children by (G desc, flat index asc);
  * the noise is drawn from a counter-based generator, SplitMix64 (Steele, Lea and
    Flood, OOPSLA 2014), keyed by (seed, request id, level, parent rank, code):
        h = sm64(sm64(seed) ^ req << 40 ^ level << 32 ^ rank << 8 ^ code)
        u = ((h >> 40) + 1/2) / 2^24,   Gumbel = -log(-log u);
  * the score returned with a beam is phi; beams are ranked by G;
  * without the SID constraint (NORM_OPEN) every code is a candidate, as in
    ``oracle.beam``.
"""
from __future__ import annotations

import math

import numpy as np

from .beam import masked_log_softmax, NORM_CHILDREN, NORM_LEVEL, NORM_OPEN

_M64 = (1 << 64) - 1


def splitmix64(x: int) -> int:
    """One SplitMix64 output for state x (Steele, Lea and Flood 2014)."""
    z = (x + 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def noise_uniform(seed: int, req: int, level: int, rank: int, code: int) -> float:
    """The uniform draw in (0, 1) for child ``code`` of the beam at ``rank``."""
    key = splitmix64(seed & _M64) ^ (req << 40) ^ (level << 32) ^ (rank << 8) ^ code
    h = splitmix64(key & _M64)
    return ((h >> 40) + 0.5) / float(1 << 24)


def gumbel(u: float) -> float:
    return -math.log(-math.log(u))


def condition_on_max(parent_key: float, z: float, g: float) -> float:
    """Key of a child with perturbed score g whose siblings' maximum z is conditioned
    to equal parent_key: -log(exp(-parent_key) - exp(-z) + exp(-g)), in the form that
    stays finite (the maximum itself gets parent_key)."""
    if g >= z:
        return float(parent_key)
    a = g - z                                     # < 0
    log1mexp = math.log(-math.expm1(a)) if a > -math.log(2.0) else math.log1p(-math.exp(a))
    v = parent_key - g + log1mexp
    return parent_key - max(v, 0.0) - math.log1p(math.exp(-abs(v)))


def expand_request_sampled(trie, depth: int, prefixes, phis, keys, logits64: np.ndarray,
                           beam_width: int, temperature: float, seed: int, req: int,
                           norm: int = NORM_CHILDREN):
    """One sampled step of one request at ``depth``.

    Rows are given in rank order by packed prefix, log-probability ``phis[r]`` and key
    ``keys[r]``; ``logits64[r]`` holds row r's logits in float64. Returns the kept
    survivors in rank order (parent, code, node, key, phi, prefix) and every candidate,
    sorted by key (cand_*)."""
    if not temperature > 0.0:
        raise ValueError("temperature must be > 0")
    V = trie.V
    ck, cphi, cflat, cpar, ccode, cnode = [], [], [], [], [], []
    for r in range(len(prefixes)):
        codes, nodes = trie.children(depth, prefixes[r])
        if norm == NORM_OPEN:                       # no constraint: every code, nodes tagged
            tagged = np.full(V, -1, dtype=np.int64)
            tagged[codes] = nodes
            codes, nodes = np.arange(V, dtype=np.int64), tagged
            logp = masked_log_softmax(logits64[r] / temperature, codes, NORM_LEVEL)
        elif codes.size == 0:
            raise ValueError("a live row sits on a node without children")
        else:
            logp = masked_log_softmax(logits64[r] / temperature, codes, norm)
        phi = float(phis[r]) + logp
        g = np.asarray([phi[i] + gumbel(noise_uniform(seed, req, depth, r, int(c)))
                        for i, c in enumerate(codes)])
        z = float(g.max())
        ck.append(np.asarray([condition_on_max(float(keys[r]), z, float(gi)) for gi in g]))
        cphi.append(phi)
        cflat.append(r * V + codes)
        cpar.append(np.full(codes.size, r, dtype=np.int64))
        ccode.append(codes)
        cnode.append(nodes)
    key = np.concatenate(ck)
    flat = np.concatenate(cflat)
    order = np.lexsort((flat, -key))
    out = {"cand_key": key[order], "cand_phi": np.concatenate(cphi)[order], "cand_flat": flat[order],
           "cand_parent": np.concatenate(cpar)[order], "cand_code": np.concatenate(ccode)[order],
           "cand_node": np.concatenate(cnode)[order]}
    k = min(int(beam_width), key.size)
    for name in ("parent", "code", "node", "key", "phi"):
        out[name] = out["cand_" + name][:k]
    pref = np.asarray([int(p) for p in prefixes], dtype=np.uint64)
    out["prefix"] = pref[out["parent"]] * np.uint64(256) + out["code"].astype(np.uint64)
    return out


def decode_sampled(trie, beam_width: int, logits_for, temperature: float, seed: int, req: int = 0,
                   norm: int = NORM_CHILDREN, n_steps=None):
    """Full sampled decode of one request (root: phi = 0, key = 0).
    ``logits_for(step, prefixes)`` returns float64 logits for the live rows."""
    n_steps = trie.L if n_steps is None else n_steps
    prefixes = np.zeros(1, dtype=np.uint64)
    phis = np.zeros(1, dtype=np.float64)
    keys = np.zeros(1, dtype=np.float64)
    history = []
    for t in range(n_steps):
        res = expand_request_sampled(trie, t, prefixes, phis, keys, logits_for(t, prefixes),
                                     beam_width, temperature, seed, req, norm)
        history.append(res)
        prefixes, phis, keys = res["prefix"], res["phi"], res["key"]
    return {"sids": prefixes, "phi": phis, "keys": keys, "history": history}
