"""Plant plausible mistakes in copies of the oracle and require that some pin fails.

Each mutant changes one thing (a dropped term, a wrong sign, a wrong index, a
transposed operand, a flipped tie-break...). A mutant that every pin accepts would
mean the pins cannot tell that mistake from the method. CPU only; nothing here
touches the HIP path.
"""
import math
import types

import numpy as np
import pytest

import oracle
from oracle import beam as ob
from oracle.trie import OracleTrie
import pins


def _expand(trie, depth, prefixes, scores, logits64, beam_width, norm=0, *, lsm=None,
            use_score=True, flat_sign=1, extra=0, score_shift=0, parent_from_code=False):
    lsm = lsm or ob.masked_log_softmax
    V = trie.V
    cs, cf, cp, cc, cn = [], [], [], [], []
    for r in range(len(prefixes)):
        codes, nodes = trie.children(depth, prefixes[r])
        logp = lsm(logits64[r], codes, norm)
        s = float(scores[(r + score_shift) % len(scores)]) if use_score else 0.0
        cs.append(s + logp)
        cf.append(r * V + codes)
        cp.append(np.full(codes.size, r))
        cc.append(codes)
        cn.append(nodes)
    score, flat = np.concatenate(cs), np.concatenate(cf)
    order = np.lexsort((flat_sign * flat, -score))
    out = {"cand_score": score[order], "cand_flat": flat[order],
           "cand_parent": np.concatenate(cp)[order], "cand_code": np.concatenate(cc)[order],
           "cand_node": np.concatenate(cn)[order]}
    k = min(beam_width + extra, score.size)
    for key in ("parent", "code", "node", "score"):
        out[key] = out["cand_" + key][:k]
    pref = np.asarray([int(p) for p in prefixes], dtype=np.uint64)
    par = out["code"] % len(pref) if parent_from_code else out["parent"]
    out["prefix"] = pref[par] * np.uint64(256) + out["code"].astype(np.uint64)
    return out


def _lsm_always(norm_forced):
    def f(x, codes, norm=0):
        return ob.masked_log_softmax(x, codes, norm_forced)
    return f


def _lsm_sign(x, codes, norm=0):
    return -ob.masked_log_softmax(x, codes, norm)


def _lsm_drop_max(x, codes, norm=0):
    support = x[codes] if norm == 0 else x
    m = support.max()
    return x[codes] - np.log(np.sum(np.exp(support - m)))


class _TrieNodeOffByOne(OracleTrie):
    def children(self, depth, prefix):
        codes, nodes = super().children(depth, prefix)
        return codes, nodes + 1


class _TrieLastRow(OracleTrie):
    def __init__(self, sids, V=256):
        super().__init__(sids, V)
        sids = np.asarray(sids)
        keys = np.zeros(sids.shape[0], dtype=np.uint64)
        for j in range(self.L):
            keys = keys * np.uint64(256) + sids[:, j].astype(np.uint64)
        rev = keys[::-1]
        _, idx = np.unique(rev, return_index=True)
        self.leaf_item = (len(keys) - 1 - idx).astype(np.int64)


class _TrieNoMask(OracleTrie):
    def children(self, depth, prefix):
        codes, nodes = super().children(depth, prefix)
        allc = np.arange(self.V, dtype=np.int64)
        fake = np.full(self.V, nodes[0] if nodes.size else 0, dtype=np.int64)
        fake[codes] = nodes
        return allc, fake


class _TrieDfsNumbering(OracleTrie):
    """Node ids in depth-first (pre-order) order instead of depth-major."""
    def __init__(self, sids, V=256):
        super().__init__(sids, V)
        order = []

        def visit(d, p):
            order.append((d, p))
            if d < self.L:
                for c in OracleTrie.children(self, d, p)[0]:
                    visit(d + 1, p * 256 + int(c))
        visit(0, 0)
        self._dfs = {dp: i for i, dp in enumerate(order)}

    def node_id(self, depth, prefix):
        return self._dfs[(depth, int(prefix))]

    def children(self, depth, prefix):
        codes, _ = super().children(depth, prefix)
        return codes, np.asarray([self._dfs[(depth + 1, int(prefix) * 256 + int(c))]
                                  for c in codes], dtype=np.int64)


def _widen_shift8(x, dtype):
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(8)
        return bits.view(np.float32).astype(np.float64)
    return ob.widen_logits(x, dtype)


def _lmhead_transposed(h, w):
    return ob.widen_logits(h, "bf16") @ ob.widen_logits(w, "bf16")


def _lmhead_f32(h, w):
    return (ob.widen_logits(h, "bf16").astype(np.float32) @
            ob.widen_logits(w, "bf16").astype(np.float32).T).astype(np.float64)


def _decode_sampled_mut(*, cond=None, gum=None, temp_mul=False, shared_noise=False,
                        parent_key=True, accumulate=True):
    """A copy of the sampled decode with one planted mistake."""
    from oracle import sample as osm
    cond = cond or osm.condition_on_max
    gum = gum or osm.gumbel

    def decode(trie, beam_width, logits_for, temperature, seed, req=0, norm=0):
        prefixes = np.zeros(1, dtype=np.uint64)
        phis, keys = np.zeros(1), np.zeros(1)
        hist = []
        for t in range(trie.L):
            x = logits_for(t, prefixes)
            V = trie.V
            ck, cphi, cflat, cpar, ccode, cnode = [], [], [], [], [], []
            for r in range(len(prefixes)):
                codes, nodes = trie.children(t, prefixes[r])
                xs = x[r] * temperature if temp_mul else x[r] / temperature
                logp = ob.masked_log_softmax(xs, codes, norm)
                phi = (float(phis[r]) if accumulate else 0.0) + logp
                g = np.asarray([phi[i] + gum(osm.noise_uniform(seed, req, t, r, 0 if shared_noise else int(c)))
                                for i, c in enumerate(codes)])
                pk = float(keys[r]) if parent_key else 0.0
                ck.append(np.asarray([cond(pk, float(g.max()), float(gi)) for gi in g]))
                cphi.append(phi)
                cflat.append(r * V + codes)
                cpar.append(np.full(codes.size, r))
                ccode.append(codes)
                cnode.append(nodes)
            key, flat = np.concatenate(ck), np.concatenate(cflat)
            order = np.lexsort((flat, -key))
            h = {"cand_key": key[order], "cand_phi": np.concatenate(cphi)[order],
                 "cand_parent": np.concatenate(cpar)[order], "cand_code": np.concatenate(ccode)[order],
                 "cand_node": np.concatenate(cnode)[order]}
            k = min(beam_width, key.size)
            for name in ("parent", "code", "node", "key", "phi"):
                h[name] = h["cand_" + name][:k]
            pref = np.asarray([int(p) for p in prefixes], dtype=np.uint64)
            prefixes = pref[h["parent"]] * np.uint64(256) + h["code"].astype(np.uint64)
            phis, keys = h["phi"], h["key"]
            hist.append(h)
        return {"sids": prefixes, "phi": phis, "keys": keys, "history": hist}
    return decode


def _exp_open_constrained(trie, depth, prefixes, scores, logits64, beam_width, norm=0):
    # open-vocabulary mode that still restricts candidates to the trie's children
    return ob.expand_request(trie, depth, prefixes, scores, logits64, beam_width, 1 if norm == 2 else norm)


def _score_mut(*, drop_level=False, reverse_levels=False, normalise=True, sid_sign=1.0,
               emb_by_item=False, tie_sign=1, lse_topk=False, extra=0, ignore_weight=False):
    """A copy of the single-pass scoring with one planted mistake."""
    from oracle import score as osc

    def score_catalog(trie, table64, k, table_kind=0, user_vec=None, sid_emb=None, sid_weight=1.0):
        codes = osc.leaf_codes(trie)
        t = np.asarray(table64, dtype=np.float64)
        logp = osc.token_log_probs(t, table_kind) if normalise else t
        L = trie.L
        score = np.zeros(trie.n_distinct)
        for j in range(L - 1 if drop_level else L):
            score += logp[j, codes[:, L - 1 - j] if reverse_levels else codes[:, j]]
        if user_vec is not None:
            emb = np.asarray(sid_emb, dtype=np.float64)
            if emb_by_item:
                emb = emb[trie.leaf_item]
            w = 1.0 if ignore_weight else float(sid_weight)
            score += sid_sign * w * (emb @ np.asarray(user_vec, dtype=np.float64))
        leaf = np.arange(score.size)
        order = np.lexsort((tie_sign * leaf, -score))
        top = order[:min(int(k) + extra, score.size)]
        pool = score[top] if lse_topk else score
        m = pool.max()
        lse = m + np.log(np.sum(np.exp(pool - m)))
        return {"leaf": top, "item": trie.leaf_item[top], "score": score[top], "lse": float(lse)}
    return score_catalog


def _sm64_wrong_multiplier(x):
    m = (1 << 64) - 1
    z = (x + 0x9E3779B97F4A7C15) & m
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B5) & m     # last digit of the first multiplier
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
    return z ^ (z >> 31)


def _noise_with(sm64, level_shift=32):
    def noise_uniform(seed, req, level, rank, code):
        m = (1 << 64) - 1
        key = sm64(seed & m) ^ (req << 40) ^ (level << level_shift) ^ (rank << 8) ^ code
        return ((sm64(key & m) >> 40) + 0.5) / float(1 << 24)
    return noise_uniform


def _ns(**over):
    ns = dict(OracleTrie=oracle.OracleTrie, expand_request=oracle.expand_request,
              masked_log_softmax=oracle.masked_log_softmax, decode=oracle.decode,
              lmhead_logits=oracle.lmhead_logits, widen_logits=oracle.widen_logits,
              decode_sampled=oracle.decode_sampled, noise_uniform=oracle.noise_uniform,
              splitmix64=oracle.splitmix64,
              gumbel=oracle.gumbel, score_catalog=oracle.score_catalog)
    ns.update(over)
    return types.SimpleNamespace(**ns)


def _exp(**kw):
    return lambda *a, **k: _expand(*a, **kw)


MUTANTS = {
    "normaliser_always_level": dict(masked_log_softmax=_lsm_always(1),
                                    expand_request=_exp(lsm=_lsm_always(1))),
    "normaliser_always_children": dict(masked_log_softmax=_lsm_always(0),
                                       expand_request=_exp(lsm=_lsm_always(0))),
    "logp_sign_flipped": dict(masked_log_softmax=_lsm_sign, expand_request=_exp(lsm=_lsm_sign)),
    "lse_dropped_max_term": dict(masked_log_softmax=_lsm_drop_max,
                                 expand_request=_exp(lsm=_lsm_drop_max)),
    "parent_score_dropped": dict(expand_request=_exp(use_score=False)),
    "parent_score_wrong_row": dict(expand_request=_exp(score_shift=1)),
    "tie_break_flat_descending": dict(expand_request=_exp(flat_sign=-1)),
    "keeps_one_extra_beam": dict(expand_request=_exp(extra=1)),
    "survivor_parent_wrong_index": dict(expand_request=_exp(parent_from_code=True)),
    "child_node_off_by_one": dict(OracleTrie=_TrieNodeOffByOne),
    "duplicate_sid_maps_to_last_row": dict(OracleTrie=_TrieLastRow),
    "children_not_masked": dict(OracleTrie=_TrieNoMask),
    "node_numbering_depth_first": dict(OracleTrie=_TrieDfsNumbering),
    "bf16_widened_wrong_shift": dict(widen_logits=_widen_shift8),
    "lmhead_operand_transposed": dict(lmhead_logits=_lmhead_transposed),
    "lmhead_fp32_accumulate": dict(lmhead_logits=_lmhead_f32),
    "open_mode_keeps_constraint": dict(expand_request=_exp_open_constrained),
    "sampled_keys_not_conditioned": dict(decode_sampled=_decode_sampled_mut(cond=lambda pk, z, g: g)),
    "sampled_gumbel_sign_flipped": dict(decode_sampled=_decode_sampled_mut(gum=lambda u: math.log(-math.log(u))),
                                        gumbel=lambda u: math.log(-math.log(u))),
    "sampled_temperature_multiplies": dict(decode_sampled=_decode_sampled_mut(temp_mul=True)),
    "sampled_noise_shared_by_siblings": dict(decode_sampled=_decode_sampled_mut(shared_noise=True)),
    "sampled_parent_key_dropped": dict(decode_sampled=_decode_sampled_mut(parent_key=False)),
    "sampled_phi_not_accumulated": dict(decode_sampled=_decode_sampled_mut(accumulate=False)),
    "splitmix_wrong_multiplier": dict(splitmix64=_sm64_wrong_multiplier,
                                      noise_uniform=_noise_with(_sm64_wrong_multiplier)),
    "noise_key_level_wrong_shift": dict(noise_uniform=_noise_with(oracle.splitmix64, level_shift=30)),
    "score_last_level_dropped": dict(score_catalog=_score_mut(drop_level=True)),
    "score_levels_reversed": dict(score_catalog=_score_mut(reverse_levels=True)),
    "score_logits_not_normalised": dict(score_catalog=_score_mut(normalise=False)),
    "score_sid_term_sign_flipped": dict(score_catalog=_score_mut(sid_sign=-1.0)),
    "score_embedding_by_catalog_row": dict(score_catalog=_score_mut(emb_by_item=True)),
    "score_tie_larger_sid_first": dict(score_catalog=_score_mut(tie_sign=-1)),
    "score_lse_over_top_k_only": dict(score_catalog=_score_mut(lse_topk=True)),
    "score_keeps_one_extra": dict(score_catalog=_score_mut(extra=1)),
    "score_sid_weight_ignored": dict(score_catalog=_score_mut(ignore_weight=True)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_rejects_mutant(name):
    ns = _ns(**MUTANTS[name])
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(ns)
        except Exception as e:          # an assertion, or the mutant breaking an invariant
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin rejects mutant {name}"
