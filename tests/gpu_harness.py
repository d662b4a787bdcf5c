"""Drive the HIP path step by step and compare every step with the oracle.

Teacher-forced: before each step the harness reads the GPU's state (row prefixes
walked back through the GPU's own back-pointers, fp32 scores) and hands exactly
that state to the oracle, so a permitted near-tie swap never changes the next
step's inputs.

Parity rule per request and step (O = the oracle's candidates best-first, k = kept
count, s_k = O's k-th score; G = the GPU's survivors, looked up in O by
(parent, code)):
  1. |G| == k
  2. every candidate whose oracle score > s_k + WIN is in G
  3. every g in G has oracle score >= s_k - WIN
  4. node(g) equals the oracle's child node and |score_gpu - score_oracle| <= TOL
  5. consecutive G entries are ordered up to WIN; exactly equal GPU scores have
     ascending flat index
  6. every position whose oracle score has no other candidate within WIN holds the
     oracle's candidate bit-exactly (parent, code, node)
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from trie_constrained_beam_amd import Beams, Trie, synth

WIN = 1e-5
TOL = 1e-4


def walk_prefixes(hist, base, rows, level):
    """Packed prefixes of rows [0, rows) of a request at ``level``, from back-pointers."""
    r = np.arange(rows, dtype=np.int64)
    key = np.zeros(rows, dtype=np.uint64)
    for lv in range(level - 1, -1, -1):
        h = hist[lv, base + r].astype(np.int64)
        key = key + (h & 255).astype(np.uint64) * (np.uint64(256) ** np.uint64(level - 1 - lv))
        r = h >> 8
    return key


def compare_step(ref, g_parent, g_code, g_node, g_score, ctx="", win=WIN, tol=TOL):
    """Apply the parity rule; returns a dict of diagnostics (near-ties seen)."""
    WIN, TOL = win, tol
    k = ref["parent"].size
    assert g_parent.size == k, f"{ctx}: kept {g_parent.size} != {k}"
    V = 256
    cand_key = ref["cand_parent"] * V + ref["cand_code"]
    pos = {int(key): i for i, key in enumerate(cand_key)}
    oscore = ref["cand_score"]
    s_k = oscore[k - 1]
    idx = []
    for j in range(k):
        key = int(g_parent[j]) * V + int(g_code[j])
        assert key in pos, f"{ctx}: survivor {j} (parent {g_parent[j]}, code {g_code[j]}) is not a candidate"
        idx.append(pos[key])
    idx = np.asarray(idx)
    assert np.unique(idx).size == k, f"{ctx}: duplicate survivors"
    # rule 2
    must = np.nonzero(oscore > s_k + WIN)[0]
    assert np.isin(must, idx).all(), f"{ctx}: a candidate clearly inside the top-k is missing"
    # rule 3
    assert (oscore[idx] >= s_k - WIN).all(), f"{ctx}: a survivor is clearly outside the top-k"
    # rule 4
    assert np.array_equal(ref["cand_node"][idx], g_node), f"{ctx}: node mismatch"
    err = np.abs(oscore[idx] - g_score.astype(np.float64))
    assert err.max(initial=0.0) <= TOL, f"{ctx}: score error {err.max()}"
    # rule 5
    os_ = oscore[idx]
    assert (os_[:-1] >= os_[1:] - WIN).all(), f"{ctx}: order violated beyond the window"
    flat = g_parent.astype(np.int64) * V + g_code
    eq = g_score[:-1] == g_score[1:]
    assert (flat[:-1][eq] < flat[1:][eq]).all(), f"{ctx}: equal scores not in flat order"
    assert (g_score[:-1] >= g_score[1:]).all(), f"{ctx}: GPU scores not non-increasing"
    # rule 6
    n = oscore.size
    lo_gap = np.full(n, np.inf)
    hi_gap = np.full(n, np.inf)
    lo_gap[1:] = oscore[:-1] - oscore[1:]
    hi_gap[:-1] = oscore[:-1] - oscore[1:]
    isolated = (lo_gap > WIN) & (hi_gap > WIN)
    iso = np.nonzero(isolated[:k])[0]
    assert np.array_equal(idx[iso], iso), f"{ctx}: an isolated position differs from the oracle"
    return {"near_ties": int(k - iso.size)}


class Run:
    """One wave on the GPU plus the matching oracle trie."""

    def __init__(self, catalog, widths, V=256, mask_depths=None, norm="children", max_slots=None,
                 max_width=None, read_mode="auto"):
        self.catalog = np.ascontiguousarray(catalog, dtype=np.uint8)
        self.widths = list(widths)
        self.trie = Trie(self.catalog, V=V, mask_depths=mask_depths, device="cuda")
        self.otrie = oracle.OracleTrie(self.catalog.astype(np.int64), V=V)
        self.V = V
        self.L = self.catalog.shape[1]
        self.norm = {"children": 0, "level": 1, "open": 2}[norm]
        self.max_slots = max_slots or int(sum(self.widths))
        self.max_width = max_width or max(self.widths)
        self.beams = Beams(self.trie, self.max_slots, len(self.widths), self.max_width, norm=norm)
        self.beams.set_read_mode(read_mode)
        self.ids, self.bases = self.beams.init(np.asarray(self.widths, dtype=np.int32))

    def state(self):
        ex = self.beams.export()
        torch.cuda.synchronize()
        return {k: v.cpu().numpy() for k, v in ex.items()}

    def step_and_check(self, t, logits_rows, dtype, stats=None, check_reqs=None):
        """``logits_rows[i]``: [rows >= live rows, V] logits of request i (f32 or bf16 bits)."""
        pre = self.state()
        S = self.max_slots
        if dtype == "f32":
            host = np.zeros((S, self.V), dtype=np.float32)
        else:
            host = np.zeros((S, self.V), dtype=np.uint16)
        for i, base in zip(range(len(self.widths)), self.bases):
            x = logits_rows[i]
            host[base:base + x.shape[0]] = x
        if dtype == "f32":
            dev = torch.from_numpy(host).cuda()
        else:
            dev = torch.from_numpy(host.view(np.int16)).cuda().view(torch.bfloat16)
        self.beams.step(dev)
        post = self.state()
        reqs = range(len(self.widths)) if check_reqs is None else check_reqs
        for i in reqs:
            rid, base = int(self.ids[i]), int(self.bases[i])
            rows = int(pre["rows"][rid])
            assert int(pre["level"][rid]) == t
            pref = walk_prefixes(pre["hist"], base, rows, t)
            scores = pre["score"][base:base + rows].astype(np.float64)
            x64 = oracle.widen_logits(logits_rows[i][:rows], dtype)
            ref = oracle.expand_request(self.otrie, t, pref, scores, x64, self.widths[i], self.norm)
            k = int(post["rows"][rid])
            h = post["hist"][t, base:base + k].astype(np.int64)
            d = compare_step(ref, h >> 8, h & 255, post["node"][base:base + k],
                             post["score"][base:base + k], ctx=f"req {i} step {t}")
            if stats is not None:
                stats["near_ties"] = stats.get("near_ties", 0) + d["near_ties"]
                stats["checked"] = stats.get("checked", 0) + 1
            assert np.array_equal(post["parent_slot"][base:base + k], base + (h >> 8))
        return post


def rowkeyed_logits(seed, t, widths, sigma, bf16):
    return [synth.logits_rowkeyed(seed, t, i, w, sigma, bf16=bf16) for i, w in enumerate(widths)]


def run_rowkeyed(catalog, widths, seed, sigma, bf16=False, mask_depths=None, norm="children",
                 check_reqs=None, read_mode="auto"):
    run = Run(catalog, widths, mask_depths=mask_depths, norm=norm, read_mode=read_mode)
    stats = {}
    for t in range(run.L):
        run.step_and_check(t, rowkeyed_logits(seed, t, widths, sigma, bf16),
                           "bf16" if bf16 else "f32", stats, check_reqs)
    return run, stats


# Sampled steps: keys pass through Gumbel noise and the conditioning logarithms in fp32,
# so the window and tolerance are wider than at temperature 0.
WIN_SAMPLED = 1e-4
TOL_SAMPLED = 3e-4


def compare_sampled_step(ref, post, base, k, level, ctx=""):
    """Parity of one sampled step: the kept set and order follow the oracle's keys (up to
    near-ties), and each survivor's key and log-probability match the oracle's."""
    h = post["hist"][level, base:base + k].astype(np.int64)
    r = dict(ref)
    r["cand_score"] = ref["cand_key"]
    d = compare_step(r, h >> 8, h & 255, post["node"][base:base + k], post["score"][base:base + k],
                     ctx=ctx, win=WIN_SAMPLED, tol=TOL_SAMPLED)
    pos = {int(p) * 256 + int(c): i for i, (p, c) in enumerate(zip(ref["cand_parent"], ref["cand_code"]))}
    idx = np.asarray([pos[int(x)] for x in (h >> 8) * 256 + (h & 255)])
    err = np.abs(ref["cand_phi"][idx] - post["phi"][base:base + k].astype(np.float64))
    assert err.max(initial=0.0) <= TOL_SAMPLED, f"{ctx}: log-probability error {err.max()}"
    return d


# Single-pass scoring: scores are sums of L fp32 table entries (|entry| <= ~70) plus an
# fp32 MFMA dot product of bf16 operands; at these magnitudes the fp32 result is within
# a few 1e-5 of the float64 oracle, so near-ties are windowed at 1e-4.
WIN_SCORE = 1e-4
TOL_SCORE = 1e-4


def compare_topk(all_scores, gpu_leaf, gpu_score, k, ctx="", win=WIN_SCORE, tol=TOL_SCORE):
    """Parity of one user's top-k against the oracle's scores of every valid SID (leaf
    order), with the windowed rules of ``compare_step``."""
    n = all_scores.size
    kk = min(k, n)
    assert (gpu_leaf[kk:] == -1).all() and np.isneginf(gpu_score[kk:]).all(), f"{ctx}: tail not empty"
    leaf = gpu_leaf[:kk].astype(np.int64)
    sc = gpu_score[:kk]
    assert leaf.min(initial=0) >= 0 and leaf.max(initial=0) < n, f"{ctx}: leaf out of range"
    assert np.unique(leaf).size == kk, f"{ctx}: duplicate leaves"
    order = np.lexsort((np.arange(n), -all_scores))
    srt = all_scores[order]
    s_k = srt[kk - 1]
    must = order[srt > s_k + win]
    assert np.isin(must, leaf).all(), f"{ctx}: a SID clearly inside the top-k is missing"
    assert (all_scores[leaf] >= s_k - win).all(), f"{ctx}: a SID clearly outside the top-k is kept"
    err = np.abs(all_scores[leaf] - sc.astype(np.float64))
    assert err.max(initial=0.0) <= tol, f"{ctx}: score error {err.max()}"
    assert (sc[:-1] >= sc[1:]).all(), f"{ctx}: scores not non-increasing"
    eq = sc[:-1] == sc[1:]
    assert (leaf[:-1][eq] < leaf[1:][eq]).all(), f"{ctx}: equal scores not in leaf order"
    os_ = all_scores[leaf]
    assert (os_[:-1] >= os_[1:] - win).all(), f"{ctx}: order violated beyond the window"
    lo = np.full(n, np.inf)
    hi = np.full(n, np.inf)
    lo[1:] = srt[:-1] - srt[1:]
    hi[:-1] = srt[:-1] - srt[1:]
    iso = np.nonzero(((lo > win) & (hi > win))[:kk])[0]
    assert np.array_equal(leaf[iso], order[iso]), f"{ctx}: an isolated position differs from the oracle"
    return int(kk - iso.size)
