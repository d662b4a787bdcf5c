"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Every check takes ``orc``, a namespace with the oracle's functions, so that
``test_oracle_mutations.py`` can run the same checks against copies of the oracle
with a planted mistake and require that some check fails.

None of these checks re-types the oracle's formula: they compare it with a
hand-derived example, closed forms, library routines on special cases
(torch.log_softmax / torch.sort, exact rational arithmetic) and with the
independent pure-Python enumerator in ``tests/bruteforce.py``.
"""
from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------- helpers
def pack(t):
    k = 0
    for c in t:
        k = k * 256 + int(c)
    return k


def unpack(k, depth):
    return tuple((int(k) >> (8 * (depth - 1 - j))) & 255 for j in range(depth))


def run_decode(orc, trie, width, logit_fn, norm=0, steps=None):
    """Decode one request with ``orc.expand_request`` step by step.

    ``logit_fn(depth, prefix_tuple)`` returns a float64 row of V logits."""
    steps = trie.L if steps is None else steps
    prefixes = np.zeros(1, dtype=np.uint64)
    scores = np.zeros(1, dtype=np.float64)
    hist = []
    for d in range(steps):
        x = np.stack([np.asarray(logit_fn(d, unpack(p, d)), dtype=np.float64) for p in prefixes])
        res = orc.expand_request(trie, d, prefixes, scores, x, width, norm)
        hist.append(res)
        prefixes, scores = res["prefix"], res["score"]
    return [unpack(p, steps) for p in prefixes], list(scores), hist


def random_catalog(rng, V, L, n):
    tuples = list(itertools.product(range(V), repeat=L))
    idx = rng.choice(len(tuples), size=min(n, len(tuples)), replace=False)
    return [tuples[i] for i in idx]


def gaussian_logit_fn(seed, V, sigma=2.0):
    cache = {}

    def f(d, p):
        key = (d, p)
        if key not in cache:
            r = np.random.default_rng([seed, d, pack(p), len(p)])
            cache[key] = r.normal(0.0, sigma, V)
        return cache[key]
    return f


# --------------------------------------------------------------------------- pins
def pin_handworked(orc):
    """Hand-derived example of tests/golden/handworked_v3_l2.json (closed forms)."""
    with open(os.path.join(GOLDEN, "handworked_v3_l2.json")) as fh:
        g = json.load(fh)
    V, L = g["V"], g["L"]
    trie = orc.OracleTrie(np.asarray(g["catalog"], dtype=np.int64), V=V)
    assert list(trie.nodes_per_depth) == g["expected_trie"]["nodes_per_depth"]
    for key, nid in g["expected_trie"]["node_of_prefix"].items():
        t = tuple(int(c) for c in key.split(",")) if key else ()
        assert trie.node_id(len(t), pack(t)) == nid, key
    for key, item in g["expected_trie"]["item_of_sid"].items():
        t = tuple(int(c) for c in key.split(","))
        assert trie.item_of(pack(t)) == item, key
    weights = {k: v for k, v in g["logit_weights_by_prefix"].items()}

    def logit_fn(d, p):
        w = weights[",".join(str(c) for c in p)]
        return [math.log(x) for x in w]
    for case in g["cases"]:
        norm = 0 if case["norm"] == "children" else 1
        sids, scores, _ = run_decode(orc, trie, case["width"], logit_fn, norm)
        exp = case["beams"]
        assert [tuple(b["sid"]) for b in exp] == sids, (case, sids)
        for b, s in zip(exp, scores):
            assert abs(s - math.log(b["p"][0] / b["p"][1])) < 1e-12
            assert trie.item_of(pack(b["sid"])) == b["item"]


def pin_trie_numbering(orc, seed=0):
    """Depth-major lexicographic node ids and child lists, against explicit enumeration."""
    rng = np.random.default_rng(seed)
    for V, L, n in [(3, 3, 12), (5, 2, 9), (4, 4, 40), (256, 3, 300)]:
        cat = [tuple(int(c) for c in rng.integers(0, V, L)) for _ in range(n)]
        trie = orc.OracleTrie(np.asarray(cat, dtype=np.int64), V=V)
        nid = 0
        for d in range(L + 1):
            prefs = sorted(set(c[:d] for c in cat))
            for p in prefs:
                assert trie.node_id(d, pack(p)) == nid
                nid += 1
            if d < L:
                for p in prefs:
                    codes, nodes = trie.children(d, pack(p))
                    kids = sorted(set(c[d] for c in cat if c[:d] == p))
                    assert list(codes) == kids
                    assert list(nodes) == [trie.node_id(d + 1, pack(p + (k,))) for k in kids]
        assert nid == sum(trie.nodes_per_depth)


def pin_dedupe_lowest_row(orc):
    cat = np.asarray([[1, 2], [0, 0], [1, 2], [0, 0], [3, 1], [1, 2]], dtype=np.int64)
    trie = orc.OracleTrie(cat, V=4)
    assert trie.n_distinct == 3
    assert trie.item_of(pack((1, 2))) == 0
    assert trie.item_of(pack((0, 0))) == 1
    assert trie.item_of(pack((3, 1))) == 4


def pin_masked_log_softmax_vs_torch(orc, seed=1):
    """Masked log-softmax equals torch.log_softmax of the masked row (library routine)."""
    rng = np.random.default_rng(seed)
    for V in (2, 7, 256):
        for _ in range(20):
            x = rng.normal(0, 3, V)
            f = int(rng.integers(1, V + 1))
            codes = np.sort(rng.choice(V, f, replace=False))
            mask = torch.zeros(V, dtype=torch.bool)
            mask[torch.from_numpy(codes)] = True
            xt = torch.from_numpy(x)
            ref_c = torch.log_softmax(xt.masked_fill(~mask, float("-inf")), 0)[mask].numpy()
            ref_l = torch.log_softmax(xt, 0)[mask].numpy()
            got_c = orc.masked_log_softmax(x, codes, 0)
            got_l = orc.masked_log_softmax(x, codes, 1)
            assert np.max(np.abs(got_c - ref_c)) < 1e-12
            assert np.max(np.abs(got_l - ref_l)) < 1e-12
            assert abs(math.fsum(np.exp(got_c)) - 1.0) < 1e-12


def pin_single_child_and_constant(orc):
    """Closed forms: a single child gets logp = 0 exactly; constant logits give -ln(fanout)."""
    # prefix 0 has one child per level; prefix 1 fans out 1 -> 3
    cat = [(0, 5, 7), (1, 2, 0), (1, 2, 1), (1, 2, 2), (1, 3, 3)]
    trie = orc.OracleTrie(np.asarray(cat), V=8)
    zero = lambda d, p: [0.0] * 8
    sids, scores, hist = run_decode(orc, trie, 8, zero)
    expect = {}
    kids = bf._children_map(cat)
    for sid in cat:
        expect[sid] = -sum(math.log(len(kids[sid[:d]])) for d in range(3))
    for sid, s in zip(sids, scores):
        assert abs(s - expect[sid]) < 1e-12, (sid, s, expect[sid])
    # ranking: descending closed-form score; exact ties by flat index (parent rank, then code)
    got = [expect[s] for s in sids]
    assert got == sorted(got, reverse=True)
    assert sids[0] == (0, 5, 7)                   # -ln 2 beats every path through prefix 1
    # after step 1 the single-child rows keep their score exactly
    h1 = hist[1]
    for par, sc in zip(h1["parent"], h1["score"]):
        if hist[0]["code"][par] == 0:
            assert sc == hist[0]["score"][par]


def pin_ties_lower_flat(orc):
    """Equal candidates: the better-ranked parent first, then the lower code."""
    cat = [(a, b) for a in range(4) for b in range(4)]
    trie = orc.OracleTrie(np.asarray(cat), V=4)
    zero = lambda d, p: [0.0] * 4
    sids, scores, _ = run_decode(orc, trie, 16, zero)
    assert sids == cat                            # all tied: flat order == lexicographic
    sids5, _, _ = run_decode(orc, trie, 5, zero)
    # step 0 keeps codes 0..3; step 1: 16 equal candidates, flat order keeps the first five
    assert sids5 == cat[:5]


def pin_full_catalog_unconstrained(orc, seed=2):
    """With every V^L tuple in the catalog the mask is a no-op, so the step is
    torch.log_softmax of each row plus a stable descending torch.sort of the flattened
    [rows*V] scores (library routines)."""
    for V, L, width in [(5, 3, 7), (16, 2, 20), (3, 4, 5)]:
        cat = list(itertools.product(range(V), repeat=L))
        trie = orc.OracleTrie(np.asarray(cat), V=V)
        fn = gaussian_logit_fn(seed, V)
        for norm in (0, 1):
            sids, scores, _ = run_decode(orc, trie, width, fn, norm)
            beams = [()]
            sc = torch.zeros(1, dtype=torch.float64)
            for d in range(L):
                x = torch.tensor(np.stack([fn(d, p) for p in beams]), dtype=torch.float64)
                cand = (sc[:, None] + torch.log_softmax(x, dim=1)).reshape(-1)
                s_sorted, idx = torch.sort(cand, descending=True, stable=True)
                k = min(width, cand.numel())
                idx = idx[:k].tolist()
                beams = [beams[i // V] + (i % V,) for i in idx]
                sc = s_sorted[:k]
            assert beams == sids
            assert np.max(np.abs(sc.numpy() - np.asarray(scores))) < 1e-12


def pin_width_one_greedy(orc, seed=3):
    """Width 1 is the greedy constrained argmax over children (closed form)."""
    rng = np.random.default_rng(seed)
    for V, L in [(6, 3), (256, 4)]:
        cat = random_catalog(rng, V, L, 60) if V < 10 else \
            [tuple(int(c) for c in rng.integers(0, V, L)) for _ in range(500)]
        trie = orc.OracleTrie(np.asarray(cat), V=V)
        fn = gaussian_logit_fn(seed + V, V)
        kids = bf._children_map(cat)
        p, total = (), 0.0
        for d in range(L):
            row = np.asarray(fn(d, p))
            ks = kids[p]
            best = max(ks, key=lambda c: (row[c], -c))
            m = max(row[k] for k in ks)
            total += row[best] - (m + math.log(sum(math.exp(row[k] - m) for k in ks)))
            p = p + (best,)
        sids, scores, _ = run_decode(orc, trie, 1, fn)
        assert sids == [p]
        assert abs(scores[0] - total) < 1e-12


def pin_wide_equals_bruteforce(orc, seed=4):
    """A beam at least as wide as every level's distinct-prefix count prunes nothing, so
    the final beams are every catalog SID ranked by summed log-probabilities."""
    rng = np.random.default_rng(seed)
    for V, L, n in [(4, 3, 30), (256, 3, 120), (7, 2, 49)]:
        cat = random_catalog(rng, V, L, n) if V ** L < 10 ** 6 else \
            [tuple(int(c) for c in rng.integers(0, V, L)) for _ in range(n)]
        trie = orc.OracleTrie(np.asarray(cat), V=V)
        width = max(trie.nodes_per_depth)
        fn = gaussian_logit_fn(seed + n, V)
        for norm in (0, 1):
            sids, scores, _ = run_decode(orc, trie, width, fn, norm)
            ref = bf.all_scores(cat, V, fn, norm)
            assert len(sids) == len(ref) == trie.n_distinct
            assert set(sids) == set(s for _, s in ref)
            d = dict((s, v) for v, s in ref)
            for s, v in zip(sids, scores):
                assert abs(v - d[s]) < 1e-12
            assert all(scores[i] >= scores[i + 1] for i in range(len(scores) - 1))


def pin_tiny_vs_replay(orc, seed=5, n_cases=150):
    """Tiny catalogs, any width, both normalisers: equal to the explicit-list replay."""
    rng = np.random.default_rng(seed)
    for case in range(n_cases):
        V = int(rng.integers(2, 6))
        L = int(rng.integers(1, 4))
        n = int(rng.integers(1, V ** L + 1))
        cat = random_catalog(rng, V, L, n)
        width = int(rng.integers(1, 9))
        norm = int(rng.integers(0, 2))
        fn = gaussian_logit_fn(seed * 1000 + case, V)
        trie = orc.OracleTrie(np.asarray(cat), V=V)
        sids, scores, _ = run_decode(orc, trie, width, fn, norm)
        ref = bf.beam_replay(cat, V, width, fn, norm)
        assert sids == [p for _, p in ref], (case, V, L, n, width, norm)
        assert np.max(np.abs(np.asarray(scores) - np.asarray([s for s, _ in ref]))) < 1e-12


def pin_legality(orc, seed=6):
    """Every emitted SID is in the catalog (illegal rate exactly 0, flashrec 0.1.0,
    Features > Decoding), no request holds a SID twice, and every survivor's node is a
    child of its parent's node."""
    rng = np.random.default_rng(seed)
    V, L = 256, 4
    cat = [tuple(int(c) for c in rng.integers(0, 8, L)) for _ in range(3000)]
    catset = set(cat)
    prefset = set(c[:d] for c in cat for d in range(L + 1))
    trie = orc.OracleTrie(np.asarray(cat), V=V)
    fn = gaussian_logit_fn(seed, V)
    sids, scores, hist = run_decode(orc, trie, 50, fn)
    assert len(sids) == 50 and len(set(sids)) == 50
    assert all(s in catset for s in sids)
    prev = [()]
    for d, h in enumerate(hist):
        cur = []
        for par, code, node in zip(h["parent"], h["code"], h["node"]):
            p = prev[par] + (int(code),)
            assert p in prefset
            assert trie.node_id(d + 1, pack(p)) == node
            pd, pp = trie.prefix_of(int(node))
            assert pd == d + 1 and pp == pack(p)
            cur.append(p)
        prev = cur


def pin_lmhead_exact(orc, seed=7):
    """fp64 H W^T from bf16 inputs equals the exact rational result; the operands have
    few significant bits, so every product and partial sum is exact in float64."""
    rng = np.random.default_rng(seed)

    # bf16 values: sign, 7 stored mantissa bits, exponent in [-8, 7]. A product has at most
    # 16 significant bits spread over 2**-16..2**15; a sum of up to 64 of them fits in 53 bits
    # (exact in float64) but not in float32's 24.
    def rand_bf16(shape):
        sign = rng.integers(0, 2, shape)
        e = rng.integers(-8, 8, shape)
        mant = rng.integers(0, 128, shape)
        val = (1 + mant / 128.0) * (2.0 ** e) * np.where(sign == 1, -1.0, 1.0)
        bits = (np.asarray(val, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
        return bits, val
    # the 4x4x4 case is square on purpose: a transposed operand still runs
    for R, V, H in [(4, 4, 4), (3, 5, 64)]:
        hb, hv = rand_bf16((R, H))
        wb, wv = rand_bf16((V, H))
        got = orc.lmhead_logits(hb, wb)
        assert got.shape == (R, V)
        for r in range(R):
            for c in range(V):
                exact = sum(Fraction(float(hv[r, k])) * Fraction(float(wv[c, k]))
                            for k in range(H))
                assert Fraction(float(got[r, c])) == exact


def pin_bf16_widening(orc):
    bits = np.asarray([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 1.0078125, 0.0, -0.0, 3.140625]
    got = orc.widen_logits(bits, "bf16")
    assert list(got) == want
    f = np.asarray([1.5, -0.25], dtype=np.float32)
    assert list(orc.widen_logits(f, "f32")) == [1.5, -0.25]


def pin_decode_api(orc, seed=8):
    """``orc.decode`` agrees with the step-by-step loop and reports catalog items."""
    rng = np.random.default_rng(seed)
    cat = [tuple(int(c) for c in rng.integers(0, 5, 3)) for _ in range(40)]
    trie = orc.OracleTrie(np.asarray(cat), V=256)
    fn = gaussian_logit_fn(seed, 256)
    sids, scores, _ = run_decode(orc, trie, 6, fn)

    def logits_for(t, prefixes):
        return np.stack([np.asarray(fn(t, unpack(p, t))) for p in prefixes])
    out = orc.decode(trie, 6, logits_for)
    assert [unpack(p, 3) for p in out["sids"]] == sids
    assert np.max(np.abs(out["scores"] - np.asarray(scores))) < 1e-12
    for p, item in zip(out["sids"], out["items"]):
        assert tuple(cat[item]) == unpack(p, 3)
        assert all(tuple(cat[j]) != unpack(p, 3) for j in range(item))


def pin_open_vocabulary(orc, seed=10):
    """Without the SID constraint the step is the plain beam search of torch.log_softmax
    over all V codes plus a stable descending torch.sort (library routines), whatever the
    catalog; a beam's node is the catalog node of its prefix, -1 once the prefix has left
    the catalog (checked against the catalog as a set); finished beams outside the
    catalog carry item -1 (flashrec 0.1.0, Evaluation: open-vocabulary engines leave a
    share of beams illegal, the constrained engine none)."""
    rng = np.random.default_rng(seed)
    for V, L, n, width in [(6, 3, 40, 9), (16, 2, 30, 12), (256, 3, 200, 20)]:
        cat = [tuple(int(c) for c in rng.integers(0, min(V, 8), L)) for _ in range(n)]
        prefset = set(c[:d] for c in cat for d in range(L + 1))
        trie = orc.OracleTrie(np.asarray(cat), V=V)
        fn = gaussian_logit_fn(seed + V, V)
        sids, scores, hist = run_decode(orc, trie, width, fn, 2)
        beams, sc = [()], torch.zeros(1, dtype=torch.float64)
        for d in range(L):
            x = torch.tensor(np.stack([fn(d, p) for p in beams]), dtype=torch.float64)
            cand = (sc[:, None] + torch.log_softmax(x, dim=1)).reshape(-1)
            s_sorted, idx = torch.sort(cand, descending=True, stable=True)
            k = min(width, cand.numel())
            beams = [beams[i // V] + (i % V,) for i in idx[:k].tolist()]
            sc = s_sorted[:k]
        assert beams == sids
        assert np.max(np.abs(sc.numpy() - np.asarray(scores))) < 1e-12
        prev = [()]
        for d, h in enumerate(hist):
            cur = [prev[p] + (int(c),) for p, c in zip(h["parent"], h["code"])]
            for p, node in zip(cur, h["node"]):
                assert (int(node) >= 0) == (p in prefset)
                if node >= 0:
                    assert trie.node_id(d + 1, pack(p)) == node
            prev = cur

        def logits_for(t, prefixes):
            return np.stack([np.asarray(fn(t, unpack(p, t))) for p in prefixes])
        out = orc.decode(trie, width, logits_for, 2)
        for p, item in zip(out["sids"], out["items"]):
            sid = unpack(p, L)
            assert (item >= 0) == (sid in set(cat))
            if item >= 0:
                assert tuple(cat[item]) == sid


# --------------------------------------------------------------------------- sampled (T > 0)
def _sampled_inclusion(orc, cat, V, logits, T, k, N, norm=0):
    """Largest z-score, over distinct SIDs, of the sampled decode's inclusion frequency
    (seeds 0..N-1) against the exact Plackett-Luce inclusion probability. Without the
    constraint (norm 2) the SIDs are every code tuple, not the catalog."""
    fn = lambda d, p: logits.get(p, [0.0] * V)
    trie = orc.OracleTrie(np.asarray(cat), V=V)
    L = len(cat[0])

    def logits_for(t, prefixes):
        return np.stack([np.asarray(fn(t, unpack(p, t)), dtype=np.float64) for p in prefixes])
    space = cat if norm != 2 else list(itertools.product(range(V), repeat=L))
    incl = bf.pl_inclusion(bf.leaf_probs(space, V, fn, T), k)
    cnt = dict.fromkeys(incl, 0)
    for seed in range(N):
        out = orc.decode_sampled(trie, k, logits_for, T, seed, 1, norm)
        sids = [unpack(p, L) for p in out["sids"]]
        assert len(sids) == min(k, len(incl)) and len(set(sids)) == len(sids)
        for s in sids:
            cnt[s] += 1
    return max(abs(cnt[s] / N - q) / math.sqrt(q * (1 - q) / N + 1e-12) for s, q in incl.items())


def pin_sampled_plackett_luce(orc):
    """Above temperature 0 the beams are a Gumbel top-k without replacement (flashrec
    0.1.0, Features > Serving, "API"): over many seeds, how often each SID is returned
    matches the exact probability that it is among k draws without replacement from the
    tempered SID distribution (Plackett-Luce, enumerated in tests/bruteforce.py)."""
    # an unbalanced three-level trie: one single-child chain, one 3 x 3 subtree
    cat = [(0, 0, 0)] + [(1, a, b) for a in range(3) for b in range(3)] + [(2, 0, 0), (2, 0, 1)]
    logits = {(): [1.5, 0.0, 0.3], (1,): [0.0, 0.2, -0.3], (1, 0): [0.1, 0.0, -0.2],
              (1, 1): [0.0, 0.4, 0.0], (1, 2): [0.3, 0.0, 0.0], (2, 0): [0.6, 0.0, 0.0]}
    assert _sampled_inclusion(orc, cat, 3, logits, 1.0, 3, 5000) < 4.5
    # two levels, temperature 0.5
    cat2 = [(0, 0), (0, 1), (0, 2), (1, 0), (2, 0), (2, 1)]
    logits2 = {(): [0.3, 1.1, -0.4, 0.0], (0,): [0.5, -0.2, 0.9, 0.0], (1,): [0.2, 0.0, 0.0, 0.0],
               (2,): [-1.0, 0.7, 0.0, 0.0]}
    assert _sampled_inclusion(orc, cat2, 4, logits2, 0.5, 2, 4000) < 4.5
    # no constraint: a partial catalog, SIDs drawn from all 3 x 3 code pairs
    logits3 = {(): [0.4, -0.3, 0.0], (0,): [0.2, 0.9, -0.5], (1,): [0.0, 0.3, 0.1], (2,): [-0.6, 0.0, 0.5]}
    assert _sampled_inclusion(orc, [(0, 1), (2, 2)], 3, logits3, 0.8, 3, 3000, norm=2) < 4.5


def pin_sampled_key_invariants(orc, seed=9):
    """Stochastic beam search invariants: among a beam's children the largest key equals
    the beam's own key exactly and no child's key exceeds it; a beam's log-probability is
    its parent's plus the child's tempered log-softmax; survivors are in key order."""
    rng = np.random.default_rng(seed)
    V, L = 256, 3
    cat = [tuple(int(c) for c in rng.integers(0, 6, L)) for _ in range(150)]
    trie = orc.OracleTrie(np.asarray(cat), V=V)
    fn = gaussian_logit_fn(seed, V)

    def logits_for(t, prefixes):
        return np.stack([np.asarray(fn(t, unpack(p, t))) for p in prefixes])
    T = 0.8
    out = orc.decode_sampled(trie, 12, logits_for, T, 1234, 5)
    prev_keys, prev_phi, prev_pref = np.zeros(1), np.zeros(1), [()]
    for d, h in enumerate(out["history"]):
        for r in range(len(prev_keys)):
            sel = h["cand_parent"] == r
            assert sel.any()
            assert h["cand_key"][sel].max() == prev_keys[r]
            assert (h["cand_key"][sel] <= prev_keys[r]).all()
            row = np.asarray(fn(d, prev_pref[r]))
            codes = h["cand_code"][sel]
            kids = sorted(set(c[d] for c in cat if c[:d] == prev_pref[r]))
            m = max(row[c] / T for c in kids)
            lse = m + math.log(math.fsum(math.exp(row[c] / T - m) for c in kids))
            want = prev_phi[r] + np.asarray([row[c] / T - lse for c in codes])
            assert np.max(np.abs(h["cand_phi"][sel] - want)) < 1e-12
        assert all(h["key"][i] >= h["key"][i + 1] for i in range(len(h["key"]) - 1))
        prev_keys, prev_phi = h["key"], h["phi"]
        prev_pref = [prev_pref[p] + (int(c),) for p, c in zip(h["parent"], h["code"])]


def pin_sampled_noise_moments(orc):
    """The per-child noise is standard Gumbel: mean = Euler's constant, variance = pi^2/6
    (closed forms), and the underlying uniforms are uniform on (0, 1)."""
    u = np.asarray([orc.noise_uniform(77, q, lv, r, c) for q in range(2) for lv in range(2)
                    for r in range(100) for c in range(256)])
    assert 0.0 < u.min() and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 0.005
    hist, _ = np.histogram(u, bins=16, range=(0.0, 1.0))
    assert hist.min() > 0.9 * u.size / 16 and hist.max() < 1.1 * u.size / 16
    g = np.asarray([orc.gumbel(x) for x in u])
    assert abs(g.mean() - 0.5772156649015329) < 0.02
    assert abs(g.var() - math.pi ** 2 / 6) < 0.05


def pin_splitmix64_known_answers(orc):
    """Known answers of the sampled step's noise stream: SplitMix64 keyed by seed,
    request, level, parent rank and code (flashrec 0.1.0, Features > Serving, "API"
    names Gumbel top-k; the generator and key layout are this repository's reading).

    * SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) seeded with 0 emits the published
      reference stream e220a8397b1dcdaf, 6e789e6aa1b965f4, 06c45d188009454f,
      f88bb8a8724c81ec, 1b39896a51a8749b; its i-th output is the mixer applied to
      i times the golden-ratio increment, which is what ``splitmix64(i * gamma)`` is.
    * The key layout is pinned through the first of those outputs: with seed 0 the
      key is sm64(0) ^ req << 40 ^ level << 32 ^ rank << 8 ^ code, so the fields
      req = 0xE220A8, level = 0x39, rank = 0x7B1DCD, code = 0xAF cancel sm64(0)
      exactly, the hashed word is sm64(0) again and u = (0xE220A8 + 1/2) / 2^24.
      A field at a wrong shift, or a wrong constant anywhere, moves u.
    """
    gamma = 0x9E3779B97F4A7C15
    stream = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F,
              0xF88BB8A8724C81EC, 0x1B39896A51A8749B]
    for i, want in enumerate(stream):
        assert orc.splitmix64((i * gamma) & ((1 << 64) - 1)) == want, i
    u = orc.noise_uniform(0, 0xE220A8, 0x39, 0x7B1DCD, 0xAF)
    assert u == (0xE220A8 + 0.5) / float(1 << 24)
    # one bit of the code flipped: the hashed word is sm64(1), a different draw
    assert orc.noise_uniform(0, 0xE220A8, 0x39, 0x7B1DCD, 0xAE) != u


# --------------------------------------------------------------------------- single-pass scoring
def _random_sids(rng, V, L, n):
    return [tuple(int(c) for c in rng.integers(0, V, L)) for _ in range(n)]


def pin_score_bruteforce(orc, seed=11):
    """Tiny catalogs (duplicates included), both table kinds, with and without the
    SID-level term, any k: equal to the pure-Python walk over all V^L tuples
    (tests/bruteforce.py), scores, ranking, log-normaliser and catalog items."""
    rng = np.random.default_rng(seed)
    for case in range(40):
        V, L = int(rng.integers(2, 6)), int(rng.integers(1, 4))
        cat = _random_sids(rng, V, L, int(rng.integers(1, V ** L + 3)))
        trie = orc.OracleTrie(np.asarray(cat), V=V)
        sids = sorted(set(cat))
        table = rng.normal(0.0, 2.0, (L, V))
        logits = bool(case % 2)
        use = case % 3 != 0
        D = int(rng.integers(1, 6))
        emb = {t: rng.normal(0.0, 1.0, D) for t in sids}
        u, w = rng.normal(0.0, 1.0, D), float(rng.normal())
        ref = bf.sprint_scores(cat, V, table, logits, u if use else None, emb, w)
        rk = bf.ranked(ref)
        k = int(rng.integers(1, len(sids) + 3))
        out = orc.score_catalog(trie, table, k, 1 if logits else 0, u if use else None,
                                np.stack([emb[t] for t in sids]) if use else None, w)
        kk = min(k, len(sids))
        assert [sids[int(l)] for l in out["leaf"]] == [t for t, _ in rk[:kk]], case
        assert np.max(np.abs(out["score"] - np.asarray([v for _, v in rk[:kk]]))) < 1e-12
        assert abs(out["lse"] - bf.log_sum_exp(list(ref.values()))) < 1e-12
        for l, it in zip(out["leaf"], out["item"]):
            assert int(it) == cat.index(sids[int(l)])


def pin_score_equals_wide_beam(orc, seed=12):
    """With position-independent logits, the level-normalised beam search at a width
    that prunes nothing ranks every valid SID by the same sum of per-position
    log-softmax terms: single-pass scoring of raw logits must give that ranking."""
    rng = np.random.default_rng(seed)
    for V, L, n in [(256, 3, 300), (6, 3, 80), (256, 2, 500)]:
        cat = _random_sids(rng, V, L, n)
        trie = orc.OracleTrie(np.asarray(cat), V=V)
        table = rng.normal(0.0, 2.0, (L, V))
        width = max(trie.nodes_per_depth)
        beams, scores, _ = run_decode(orc, trie, width, lambda d, p: table[d], norm=1)
        out = orc.score_catalog(trie, table, trie.n_distinct, 1)
        sids = sorted(set(cat))
        assert [sids[int(l)] for l in out["leaf"]] == beams
        assert np.max(np.abs(out["score"] - np.asarray(scores))) < 1e-12


def pin_score_full_catalog(orc, seed=13):
    """Every V^L tuple valid: the token distributions multiply to a distribution over
    the product space, so the log-normaliser is 0; the best k equal a stable
    descending torch.sort of the outer sum of torch.log_softmax rows."""
    rng = np.random.default_rng(seed)
    V, L, k = 16, 3, 50
    cat = list(itertools.product(range(V), repeat=L))
    perm = rng.permutation(len(cat))
    cat = [cat[i] for i in perm]                       # catalog rows != leaf order
    trie = orc.OracleTrie(np.asarray(cat), V=V)
    table = rng.normal(0.0, 3.0, (L, V))
    lp = torch.log_softmax(torch.tensor(table, dtype=torch.float64), dim=1)
    total = (lp[0][:, None, None] + lp[1][None, :, None] + lp[2][None, None, :]).reshape(-1)
    s_sorted, idx = torch.sort(total, descending=True, stable=True)
    for kind, tab in ((1, table), (0, lp.numpy())):
        out = orc.score_catalog(trie, tab, k, kind)
        assert abs(out["lse"]) < 1e-12
        assert out["leaf"].tolist() == idx[:k].tolist()
        assert np.max(np.abs(out["score"] - s_sorted[:k].numpy())) < 1e-12
        inv = np.argsort(perm)
        assert out["item"].tolist() == [int(inv[l]) for l in out["leaf"]]


def pin_score_sid_term_closed_form(orc, seed=14):
    """Zero token table and one-hot SID embeddings (leaf l -> 2 e_(l mod 8)): the
    matrix product reduces to a lookup, score(l) = 2 w u[l mod 8], and the
    log-normaliser is log sum over residues r of count_r exp(2 w u[r])."""
    rng = np.random.default_rng(seed)
    V, L, D, w = 256, 2, 8, 0.75
    trie = orc.OracleTrie(np.asarray(_random_sids(rng, V, L, 400)), V=V)
    n = trie.n_distinct
    emb = np.zeros((n, D))
    emb[np.arange(n), np.arange(n) % D] = 2.0
    u = rng.permutation(D).astype(np.float64) - 3.5
    out = orc.score_catalog(trie, np.zeros((L, V)), 37, 0, u, emb, w)
    expect = sorted(range(n), key=lambda l: (-2 * w * u[l % D], l))[:37]
    assert out["leaf"].tolist() == expect
    assert np.max(np.abs(out["score"] - 2 * w * u[np.asarray(expect) % D])) < 1e-12
    cnt = np.bincount(np.arange(n) % D, minlength=D)
    lse = math.log(math.fsum(float(cnt[r]) * math.exp(2 * w * u[r]) for r in range(D)))
    assert abs(out["lse"] - lse) < 1e-12


def pin_score_invariances(orc, seed=15):
    """A per-position constant added to raw logits changes nothing; added to
    log-probabilities it shifts every score and the log-normaliser by the constants'
    sum. A constant table ties every SID: the k smallest SIDs win, and the
    log-normaliser is log n + L c."""
    rng = np.random.default_rng(seed)
    V, L = 256, 3
    trie = orc.OracleTrie(np.asarray(_random_sids(rng, V, L, 2000)), V=V)
    table = rng.normal(0.0, 2.0, (L, V))
    c = rng.normal(0.0, 5.0, L)
    a, b = orc.score_catalog(trie, table, 100, 1), orc.score_catalog(trie, table + c[:, None], 100, 1)
    assert a["leaf"].tolist() == b["leaf"].tolist()
    assert np.max(np.abs(a["score"] - b["score"])) < 1e-11 and abs(a["lse"] - b["lse"]) < 1e-11
    a, b = orc.score_catalog(trie, table, 100, 0), orc.score_catalog(trie, table + c[:, None], 100, 0)
    assert a["leaf"].tolist() == b["leaf"].tolist()
    assert np.max(np.abs(b["score"] - a["score"] - c.sum())) < 1e-11
    assert abs(b["lse"] - a["lse"] - c.sum()) < 1e-11
    out = orc.score_catalog(trie, np.full((L, V), -1.25), 64, 0)
    assert out["leaf"].tolist() == list(range(64))
    assert abs(out["lse"] - (math.log(trie.n_distinct) - 1.25 * L)) < 1e-11


ALL_PINS = [pin_handworked, pin_trie_numbering, pin_dedupe_lowest_row,
            pin_masked_log_softmax_vs_torch, pin_single_child_and_constant, pin_ties_lower_flat,
            pin_full_catalog_unconstrained, pin_width_one_greedy, pin_wide_equals_bruteforce,
            pin_tiny_vs_replay, pin_legality, pin_lmhead_exact, pin_bf16_widening,
            pin_decode_api, pin_open_vocabulary, pin_sampled_plackett_luce, pin_sampled_key_invariants,
            pin_sampled_noise_moments, pin_splitmix64_known_answers, pin_score_bruteforce, pin_score_equals_wide_beam,
            pin_score_full_catalog, pin_score_sid_term_closed_form, pin_score_invariances]
