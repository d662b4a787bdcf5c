"""Single-pass scoring of every valid SID, written plainly in float64.
Test infrastructure only.

SPRINT summary (method and inference paragraphs): one forward pass gives, per user,
an L-by-M table of per-position token distributions (M = the codebook size, V = 256
here) and a user vector. Only SIDs that are valid in a prefix trie of the catalog are
scored; a SID's score is the sum of its tokens' log-probabilities plus a SID-level
similarity, which the page describes as a table lookup plus one matrix product, and
the K best SIDs are returned. Inference softmaxes over the set of valid SIDs.

Readings taken where the page is silent (each also listed in the design doc):
  * the table holds either log-probabilities (used as they are) or raw per-position
    logits, which are normalised by a log-softmax over the V codes of each position;
  * the SID-level similarity is w * <u, e_s>: u the user vector, e_s one embedding
    row per valid SID (leaf order, i.e. ascending SID), both bfloat16, w a scalar;
    the products are exact in float64;
  * the ranking is (score descending, leaf ascending): the smaller SID wins a tie;
  * the softmax over valid SIDs is returned as its log-normaliser
    lse = log sum over valid s of exp(score_s), so P(s) = exp(score_s - lse);
  * K larger than the number of valid SIDs returns every SID.
"""
from __future__ import annotations

import numpy as np

TABLE_LOGPROB = 0
TABLE_LOGITS = 1


def leaf_codes(trie) -> np.ndarray:
    """[n_distinct, L] codes of the trie's leaves in leaf (ascending SID) order."""
    out = np.zeros((trie.n_distinct, trie.L), dtype=np.int64)
    for j in range(trie.L):
        shift = np.uint64(8 * (trie.L - 1 - j))
        out[:, j] = ((trie.leaf_keys >> shift) & np.uint64(255)).astype(np.int64)
    return out


def token_log_probs(table64: np.ndarray, table_kind: int) -> np.ndarray:
    """[L, V] per-position log-probabilities from the user's table."""
    t = np.asarray(table64, dtype=np.float64)
    if table_kind == TABLE_LOGPROB:
        return t
    if table_kind != TABLE_LOGITS:
        raise ValueError(table_kind)
    m = t.max(axis=1, keepdims=True)
    return t - (m + np.log(np.sum(np.exp(t - m), axis=1, keepdims=True)))


def sid_scores(trie, table64, table_kind=TABLE_LOGPROB, user_vec=None, sid_emb=None,
               sid_weight=1.0) -> np.ndarray:
    """Score of every valid SID (leaf order) for one user."""
    codes = leaf_codes(trie)
    logp = token_log_probs(table64, table_kind)
    score = np.zeros(trie.n_distinct, dtype=np.float64)
    for j in range(trie.L):
        score += logp[j, codes[:, j]]
    if user_vec is not None:
        emb = np.asarray(sid_emb, dtype=np.float64)
        if emb.shape[0] != trie.n_distinct:
            raise ValueError("one SID embedding row per valid SID")
        score += float(sid_weight) * (emb @ np.asarray(user_vec, dtype=np.float64))
    return score


def score_catalog(trie, table64, k, table_kind=TABLE_LOGPROB, user_vec=None, sid_emb=None,
                  sid_weight=1.0):
    """Top-k valid SIDs of one user: leaf ids, catalog items, scores, and the
    log-normaliser of the softmax over all valid SIDs."""
    score = sid_scores(trie, table64, table_kind, user_vec, sid_emb, sid_weight)
    leaf = np.arange(score.size, dtype=np.int64)
    order = np.lexsort((leaf, -score))
    top = order[:min(int(k), score.size)]
    m = score.max()
    lse = m + np.log(np.sum(np.exp(score - m)))
    return {"leaf": top, "item": trie.leaf_item[top], "score": score[top], "lse": float(lse),
            "all_scores": score, "order": order}
