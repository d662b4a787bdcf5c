"""The constrained wide-beam step, written plainly in float64. Test infrastructure only.

One step of one request (flashrec 0.1.0, Features > Decoding; OneLA summary,
sections 2.1 and 3.3):
  1. every live beam row r, whose trie node is prefix p_r at depth t, may only be
     continued by the children K_r of p_r (illegal SIDs are never candidates);
  2. its logits over the level's code range are masked to K_r and log-softmaxed:
     logp_{r,c} = x_{r,c} - (m_r + ln sum_{c' in K_r} exp(x_{r,c'} - m_r)),
     m_r = max_{c' in K_r} x_{r,c'};
  3. the candidate (r, c) scores s_r + logp_{r,c} (summed token log-probabilities);
  4. the request keeps its best min(n, #candidates) candidates, n = beam width,
     chosen over all (row, child) pairs at once;
  5. survivor j records its parent row r and code c; its node is the child node.

Readings taken where the pages are silent (each also listed in the design doc):
  * normaliser (step 2): the children of the row's node (NORM_CHILDREN). The pages
    say the logits are restricted to valid continuations before scoring; SPRINT
    softmaxes over the valid set. NORM_LEVEL (all V codes of the level, then mask)
    is kept as a flag for the codebook-range reading.
  * order (step 4): score descending, then flat index r*V + c ascending, so equal
    scores go to the better-ranked parent, then the lower code. -0.0 equals +0.0.
  * survivors are emitted in that rank order, and the next step's rows follow it.
  * start: one root row with score 0; fewer candidates than n: all survive.
  * no temperature, no length penalty (temperature 0, fixed depth).
"""
from __future__ import annotations

import numpy as np

NORM_CHILDREN = 0
NORM_LEVEL = 1
# No SID constraint (the open-vocabulary comparison of flashrec 0.1.0, Evaluation, where
# engines without the constraint leave a share of beams outside the catalog): every code
# of the level is a candidate, normalised over all V codes; the trie only tags a beam's
# node, -1 once its prefix has left the catalog.
NORM_OPEN = 2


# --------------------------------------------------------------------------- inputs
def widen_logits(x, dtype: str) -> np.ndarray:
    """Logits to float64 exactly: float32 values, or bfloat16 bit patterns (uint16)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def lmhead_logits(hidden_bf16, weight_bf16) -> np.ndarray:
    """SID-range lm_head (flashrec 0.1.0, Features > Decoding: lm_head only over the
    SID token range): X = H W^T in float64 from bfloat16 hidden [R, H] and weight [V, H].
    No bias and no scale (reading). Products of bf16 values are exact in float64."""
    h = widen_logits(hidden_bf16, "bf16")
    w = widen_logits(weight_bf16, "bf16")
    return h @ w.T


# --------------------------------------------------------------------------- step
def masked_log_softmax(x_row: np.ndarray, codes: np.ndarray, norm: int = NORM_CHILDREN):
    """log-probabilities of ``codes`` under the masked log-softmax of one row (float64)."""
    support = x_row[codes] if norm == NORM_CHILDREN else x_row
    m = support.max()
    lse = m + np.log(np.sum(np.exp(support - m)))
    return x_row[codes] - lse


def expand_request(trie, depth: int, prefixes, scores, logits64: np.ndarray,
                   beam_width: int, norm: int = NORM_CHILDREN):
    """One constrained beam step of one request at ``depth`` (0-based level).

    ``prefixes[r]`` (packed) and ``scores[r]`` describe live row r, in rank order;
    ``logits64[r]`` is row r's logits over the level's V codes, widened to float64.
    With ``norm == NORM_OPEN`` every code is a candidate and a node is -1 off the catalog.
    Returns a dict of numpy arrays:
      cand_*   every candidate, sorted best-first (score, flat, parent, code, node)
      parent, code, node, score, prefix   the kept survivors, in rank order
    """
    V = trie.V
    R = len(prefixes)
    c_score, c_flat, c_par, c_code, c_node = [], [], [], [], []
    for r in range(R):
        codes, nodes = trie.children(depth, prefixes[r])
        if norm == NORM_OPEN:
            tagged = np.full(V, -1, dtype=np.int64)
            tagged[codes] = nodes
            codes, nodes = np.arange(V, dtype=np.int64), tagged
            logp = masked_log_softmax(logits64[r], codes, NORM_LEVEL)
        elif codes.size == 0:
            raise ValueError("a live row sits on a node without children")
        else:
            logp = masked_log_softmax(logits64[r], codes, norm)
        c_score.append(float(scores[r]) + logp)
        c_flat.append(r * V + codes)
        c_par.append(np.full(codes.size, r, dtype=np.int64))
        c_code.append(codes)
        c_node.append(nodes)
    score = np.concatenate(c_score)
    flat = np.concatenate(c_flat)
    order = np.lexsort((flat, -score))          # score descending, then flat ascending
    out = {
        "cand_score": score[order], "cand_flat": flat[order],
        "cand_parent": np.concatenate(c_par)[order], "cand_code": np.concatenate(c_code)[order],
        "cand_node": np.concatenate(c_node)[order],
    }
    k = min(int(beam_width), score.size)
    for key in ("parent", "code", "node", "score"):
        out[key] = out["cand_" + key][:k]
    pref = np.asarray([int(p) for p in prefixes], dtype=np.uint64)
    out["prefix"] = pref[out["parent"]] * np.uint64(256) + out["code"].astype(np.uint64)
    return out


# --------------------------------------------------------------------------- decode
def decode(trie, beam_width: int, logits_for, norm: int = NORM_CHILDREN, n_steps=None):
    """Full L-step decode of one request.

    ``logits_for(step, prefixes)`` returns float64 logits [len(prefixes), V] for the
    live rows (given by their packed prefixes, in rank order).
    Returns the final beams ranked best-first: packed SIDs, float64 scores, items.
    """
    n_steps = trie.L if n_steps is None else n_steps
    prefixes = np.zeros(1, dtype=np.uint64)
    scores = np.zeros(1, dtype=np.float64)
    history = []
    for t in range(n_steps):
        x = logits_for(t, prefixes)
        res = expand_request(trie, t, prefixes, scores, x, beam_width, norm)
        history.append(res)
        prefixes, scores = res["prefix"], res["score"]
    items = (np.asarray([trie.item_of(p) if trie.contains(p) else -1 for p in prefixes], dtype=np.int64)
             if n_steps == trie.L else None)
    return {"sids": prefixes, "scores": scores, "items": items, "history": history}
