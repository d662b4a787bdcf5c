"""CPU oracle for the catalog-constrained wide-beam expansion step.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The product path (``trie_constrained_beam_amd`` and its HIP library) never does,
and shares no code with it: the oracle builds its own trie, does its own
arithmetic in float64 and sorts with numpy.

What it computes, and where the pages say so:
  * the trie restricts every continuation to valid catalog SIDs, so an illegal SID
    is never a candidate (flashrec 0.1.0, Features > Decoding, "SID constraint");
  * each beam's score is the sum of token log-probabilities (SPRINT summary,
    inference paragraph: a SID is scored by the sum of its tokens' log-probabilities; flashrec 0.1.0, Quickstart:
    beams are returned ranked best-first with a sequence score);
  * selection is deterministic top-k at temperature 0, and a Gumbel top-k without
    replacement above it (flashrec 0.1.0, Features > Serving, "API"; ``oracle.sample``);
  * candidates are selected globally over all (beam, child) pairs of a request
    (OneLA summary, section 2.1), and survivors keep only an index to their parent
    (OneLA summary, sections 2.4 and 3.3);
  * rows of different requests share a step but never compete (flashrec 0.1.0,
    Features > Decoding, "Scheduling");
  * single-pass scoring: every valid SID is scored from a per-user table of token
    log-probabilities plus a SID-level similarity, then the top K are kept (SPRINT
    summary, method and inference paragraphs; ``oracle.score``).

Readings of points the pages leave open are listed in the module docstrings of
``oracle.beam``. Pins: ``tests/test_oracle_pins.py`` and ``tests/golden/``.
"""
from .trie import OracleTrie
from .beam import (widen_logits, masked_log_softmax, expand_request, decode,
                   lmhead_logits, NORM_CHILDREN, NORM_LEVEL, NORM_OPEN)
from .sample import (splitmix64, noise_uniform, gumbel, condition_on_max,
                     expand_request_sampled, decode_sampled)
from .score import (leaf_codes, token_log_probs, sid_scores, score_catalog, TABLE_LOGPROB,
                    TABLE_LOGITS)

__all__ = ["OracleTrie", "widen_logits", "masked_log_softmax", "expand_request",
           "decode", "lmhead_logits", "NORM_CHILDREN", "NORM_LEVEL", "NORM_OPEN", "splitmix64",
           "noise_uniform", "gumbel", "condition_on_max", "expand_request_sampled",
           "decode_sampled", "leaf_codes", "token_log_probs", "sid_scores", "score_catalog",
           "TABLE_LOGPROB", "TABLE_LOGITS"]
