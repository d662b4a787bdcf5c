"""Pure-Python enumeration for tiny catalogs: an implementation independent of ``oracle/``.

It shares nothing with the oracle: prefixes are Python tuples kept in sets and
dicts, the log-softmax uses ``math``, and ordering uses Python's ``sorted``.

* ``all_scores`` scores every distinct catalog SID by its summed per-level
  log-probabilities (SPRINT summary, inference paragraph: the token
  log-probability sum over valid SIDs of a prefix trie). A beam at least as wide
  as the number of distinct prefixes at every depth never prunes, so its final
  beams must equal this list.
* ``beam_replay`` replays the constrained beam search by listing every
  (row, child) candidate of a step explicitly and sorting the list.
"""
from __future__ import annotations

import math

CHILDREN, LEVEL = 0, 1


def _children_map(catalog):
    kids = {}
    for sid in catalog:
        for d in range(len(sid)):
            kids.setdefault(tuple(sid[:d]), set()).add(sid[d])
    return {p: sorted(s) for p, s in kids.items()}


def _logp(row, support, code):
    m = max(row[c] for c in support)
    lse = m + math.log(math.fsum(math.exp(row[c] - m) for c in support))
    return row[code] - lse


def all_scores(catalog, V, logit_fn, norm=CHILDREN):
    """[(score, sid)] for every distinct SID, best first (ties: smaller SID first)."""
    kids = _children_map(catalog)
    out = []
    for sid in sorted(set(tuple(s) for s in catalog)):
        total = 0.0
        for d in range(len(sid)):
            p = tuple(sid[:d])
            row = logit_fn(d, p)
            support = kids[p] if norm == CHILDREN else range(V)
            total += _logp(row, support, sid[d])
        out.append((total, sid))
    out.sort(key=lambda t: (-t[0], t[1]))
    return out


def beam_replay(catalog, V, width, logit_fn, norm=CHILDREN, steps=None):
    """Constrained beam search by explicit candidate lists; returns [(score, sid)] ranked."""
    kids = _children_map(catalog)
    L = len(catalog[0])
    steps = L if steps is None else steps
    beams = [(0.0, ())]
    for d in range(steps):
        cands = []
        for r, (s, p) in enumerate(beams):
            row = logit_fn(d, p)
            support = kids[p] if norm == CHILDREN else range(V)
            for c in kids[p]:
                cands.append((s + _logp(row, support, c), r * V + c, p + (c,)))
        cands.sort(key=lambda t: (-t[0], t[1]))
        beams = [(s, p) for s, _, p in cands[:width]]
    return beams


def leaf_probs(catalog, V, logit_fn, temperature):
    """{sid: probability} of every distinct SID when each level picks a child of the
    prefix with probability softmax(x / T) over the prefix's children (math module)."""
    kids = _children_map(catalog)
    out = {}
    for sid in sorted(set(tuple(s) for s in catalog)):
        lp = 0.0
        for d in range(len(sid)):
            row = [v / temperature for v in logit_fn(d, tuple(sid[:d]))]
            lp += _logp(row, kids[tuple(sid[:d])], sid[d])
        out[sid] = math.exp(lp)
    return out


def pl_inclusion(probs, k):
    """Probability that each item is among k draws without replacement, each draw
    picking a remaining item with probability proportional to its weight (explicit
    enumeration of the ordered draws)."""
    items = list(probs)
    incl = {s: 0.0 for s in items}

    def rec(chosen, p_seq, rest_mass):
        if len(chosen) == k or len(chosen) == len(items):
            for s in chosen:
                incl[s] += p_seq
            return
        for s in items:
            if s not in chosen:
                rec(chosen + [s], p_seq * probs[s] / rest_mass, rest_mass - probs[s])
    rec([], 1.0, math.fsum(probs.values()))
    return incl


def sprint_scores(catalog, V, table, table_logits, user_vec=None, emb=None, weight=1.0):
    """{sid: score} for every valid SID of a tiny catalog, found by walking all V^L
    tuples and keeping those in the catalog (math module only).

    Score = sum over positions of the token log-probability (``table[j]`` itself, or
    its log-softmax over the V codes when ``table_logits``) plus ``weight`` times the
    dot product of ``user_vec`` with ``emb[sid]`` (a dict keyed by SID tuple)."""
    import itertools
    valid = set(tuple(int(c) for c in s) for s in catalog)
    L = len(next(iter(valid)))
    logp = []
    for j in range(L):
        row = [float(v) for v in table[j]]
        if table_logits:
            lse = _logp(row, range(V), 0) - row[0]          # -(log-sum-exp of the row)
            row = [v + lse for v in row]
        logp.append(row)
    out = {}
    for t in itertools.product(range(V), repeat=L):
        if t not in valid:
            continue
        s = math.fsum(logp[j][t[j]] for j in range(L))
        if user_vec is not None:
            s += weight * math.fsum(float(a) * float(b) for a, b in zip(user_vec, emb[t]))
        out[t] = s
    return out


def ranked(scores):
    """[(sid, score)] best first; the smaller SID wins a tie."""
    return sorted(scores.items(), key=lambda kv: (-kv[1], kv[0]))


def log_sum_exp(values):
    m = max(values)
    return m + math.log(math.fsum(math.exp(v - m) for v in values))
