"""FIFO admission of requests into one decode wave under a beam-row slot budget.

flashrec 0.1.0, Features > Decoding ("Scheduling"): requests are admitted into decode
waves between steps while their beam rows fit a slot budget, and every admitted request
advances one level per step. The admission order the pages leave open is taken as FIFO
by request index, all requests arriving at once: between two steps the finished
requests are finalized (their slots return to the pool), then queued requests are
admitted in order until the next one does not fit; a request is never skipped.

This module only schedules: every step of the beam path runs in libtcb.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional

from ._lib import TcbError
from .api import Beams

TCB_E_BUDGET = -3


class WaveRequest:
    __slots__ = ("index", "width", "rid", "base", "level")

    def __init__(self, index: int, width: int):
        self.index, self.width = index, width
        self.rid = self.base = -1
        self.level = 0


def run_wave(beams: Beams, widths: List[int],
             step_fn: Callable[[int, List[WaveRequest]], None],
             on_finalize: Optional[Callable[[List[WaveRequest], dict], None]] = None) -> Dict[int, dict]:
    """Decode every request of ``widths`` through ``beams`` with FIFO admission.

    ``step_fn(step, live)`` must run exactly one beam step (``beams.step`` or
    ``beams.step_lmhead``) for the live requests ``live`` (admitted, unfinished; each
    with its slot ``base`` and current ``level``). Returns, per request index, the
    finalized result: ``sids`` [count, L], ``scores``, ``items``.
    """
    L = beams.trie.L
    queue = [WaveRequest(i, int(w)) for i, w in enumerate(widths)]
    for q in queue:
        if q.width > beams.max_slots or q.width > beams.max_width:
            raise ValueError(f"request {q.index} of width {q.width} can never be admitted")
    head, live, results, step = 0, [], {}, 0
    while head < len(queue) or live:
        # admit in order while the next request fits
        st = beams.status()
        take = []
        free, free_ids = st["free_slots"], st["free_requests"]
        while head + len(take) < len(queue):
            q = queue[head + len(take)]
            if q.width > free or free_ids == 0:
                break
            take.append(q)
            free -= q.width
            free_ids -= 1
        rids, bases = [], []
        while take:
            try:
                rids, bases = beams.init([q.width for q in take])
                break
            except TcbError as e:              # fragmented slots: admit fewer this time
                if e.code != TCB_E_BUDGET:
                    raise
                take.pop()
        for q, rid, base in zip(take, rids, bases):
            q.rid, q.base, q.level = int(rid), int(base), 0
            live.append(q)
        head += len(take)
        if not live:
            raise RuntimeError("no request fits the wave")
        step_fn(step, list(live))
        step += 1
        for q in live:
            q.level += 1
        done = [q for q in live if q.level >= L]
        if done:
            out = beams.finalize([q.rid for q in done])
            for k, q in enumerate(done):
                c = int(out["counts"][k])
                results[q.index] = {"sids": out["sids"][k, :c].copy(), "scores": out["scores"][k, :c].copy(),
                                    "items": out["items"][k, :c].copy()}
            if on_finalize is not None:
                on_finalize(done, out)
            live = [q for q in live if q.level < L]
    return results
