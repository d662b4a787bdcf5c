"""Requests finished inside the step that completes them (tcb_beams_set_finish_outputs)
against the separate finalize pass on the same seeded inputs: the outputs must be bitwise
equal, and the finishing step must release the requests' ids and slots. The finalize pass
itself is checked against the oracle step by step in test_gpu_parity.py; the cases here
reach every route of the finishing step: the merge kernel's on-chip walk of the
back-pointers (rows <= 1024), its walk from memory (wider beams), the merge inside the tile
kernel (beams of at most 64 rows), the exact selection paths under ties, sampled steps,
the unconstrained wave, a one-level catalog, the lm_head step and requests admitted
mid-decode into released slots.
"""
import numpy as np
import pytest
import torch

from trie_constrained_beam_amd import Beams, Trie, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    print(f"\n[gpu] {request.node.name}", flush=True)


def _decode(trie, widths, logits_fn, finish, norm="children", temperature=0.0, bf16=False, max_slots=None):
    """One full decode of `widths`; returns the per-request results (in `widths` order)."""
    S = max_slots or int(sum(widths))
    R, B, L = len(widths), max(widths), trie.L
    beams = Beams(trie, S, R, B, norm=norm)
    out = beams.set_finish_outputs(True) if finish else None
    ids, bases = beams.init(np.asarray(widths, dtype=np.int32))
    for t in range(L):
        host = np.zeros((S, 256), dtype=np.float32)
        for i, (w, b) in enumerate(zip(widths, bases)):
            host[b:b + w] = logits_fn(t, i, w)
        x = torch.from_numpy(host).cuda()
        if bf16:
            x = x.to(torch.bfloat16)
        beams.step(x, temperature=temperature, seed=1000 + t)
    if finish:
        torch.cuda.synchronize()
        res = {k: v.cpu().numpy()[np.asarray(ids)] for k, v in out.items()}
        st = beams.status()
        assert st["finished"] == 0 and st["active"] == 0, st
        assert st["free_slots"] == S and st["free_requests"] == R, st
    else:
        res = beams.finalize(ids)
    beams.check()
    return res


def _same(a, b):
    for k in ("counts", "sids", "scores", "items"):
        assert np.array_equal(a[k], b[k]), k


def _rowkeyed(seed, sigma=2.0):
    return lambda t, i, w: synth.logits_rowkeyed(seed, t, i, w, sigma)


CASES = {
    # name: (catalog args, widths, seed, norm, temperature, bf16)
    "merge_kernel_onchip_walk": ((100_000, 4, ("zipf",) * 4, [61, 1]), [512, 300, 64, 1, 77], 61, "children", 0.0,
                                 False),
    "merge_kernel_bf16": ((200_000, 4, ("zipf",) * 4, [62, 1]), [512] * 3, 62, "children", 0.0, True),
    "merge_kernel_walk_from_memory": ((100_000, 4, ("zipf",) * 4, [63, 1]), [2000, 5], 63, "children", 0.0, False),
    "in_tile_merge": ((100_000, 4, ("zipf",) * 4, [64, 1]), [64, 33, 1, 50], 64, "children", 0.0, False),
    "sampled": ((100_000, 4, ("zipf",) * 4, [65, 1]), [512, 40], 65, "children", 0.7, False),
    "open": ((50_000, 4, ("zipf",) * 4, [66, 1]), [256, 20], 66, "open", 0.0, False),
    "level_norm_l5": ((300_000, 5, ("uniform",) + ("zipf",) * 4, [67, 1]), [128, 512, 9], 67, "level", 0.0, False),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_finish_in_step_matches_finalize(name):
    cat_args, widths, seed, norm, temp, bf16 = CASES[name]
    trie = Trie(synth.catalog(*cat_args), device="cuda")
    fn = _rowkeyed(seed)
    a = _decode(trie, widths, fn, True, norm=norm, temperature=temp, bf16=bf16)
    b = _decode(trie, widths, fn, False, norm=norm, temperature=temp, bf16=bf16)
    _same(a, b)
    assert list(a["counts"]) == [min(w, int(c)) for w, c in zip(widths, b["counts"])]


def test_finish_under_exact_ties():
    """Constant logits: every step is a tie broken by flat index, and the wide requests'
    tiles and merges take their exact selection paths."""
    a, b_, c = np.meshgrid(np.arange(256), np.arange(256), np.arange(4), indexing="ij")
    trie = Trie(np.stack([a.ravel(), b_.ravel(), c.ravel()], axis=1).astype(np.uint8), device="cuda")
    zero = lambda t, i, w: np.zeros((w, 256), dtype=np.float32)
    for widths in ([300, 64, 7], [64, 17]):
        _same(_decode(trie, widths, zero, True), _decode(trie, widths, zero, False))


def test_finish_one_level_catalog():
    trie = Trie(np.arange(200, dtype=np.uint8).reshape(-1, 1), device="cuda")
    fn = _rowkeyed(68)
    for widths in ([50, 256], [300, 1]):
        a = _decode(trie, widths, fn, True)
        _same(a, _decode(trie, widths, fn, False))
        assert (a["items"][0, :int(a["counts"][0])] == a["sids"][0, :int(a["counts"][0]), 0]).all()


def test_finish_lmhead_step():
    cat = synth.catalog(60_000, 3, ("zipf",) * 3, [69, 1])
    trie = Trie(cat, device="cuda")
    widths, H = [512, 100, 20], 256
    S, R, B = sum(widths), len(widths), max(widths)
    w_dev = torch.from_numpy(np.stack([synth.lmhead_weight(69, lv, 256, H) for lv in range(3)]).view(np.int16))
    w_dev = w_dev.cuda().view(torch.bfloat16)
    hidden = [torch.from_numpy(synth.hidden_states(69, t, S, H).view(np.int16)).cuda().view(torch.bfloat16)
              for t in range(3)]
    res = []
    for finish in (True, False):
        beams = Beams(trie, S, R, B)
        out = beams.set_finish_outputs(True) if finish else None
        ids, _ = beams.init(np.asarray(widths, dtype=np.int32))
        for t in range(3):
            beams.step_lmhead(hidden[t], w_dev)
        if finish:
            torch.cuda.synchronize()
            res.append({k: v.cpu().numpy()[np.asarray(ids)] for k, v in out.items()})
        else:
            res.append(beams.finalize(ids))
        beams.check()
    _same(res[0], res[1])


def test_finish_mid_decode_admission_and_reuse():
    """Requests admitted between steps finish in different steps; each finishing step
    releases its requests, whose ids and slots the next admission reuses (their output
    rows are then overwritten when the new requests finish). Every request's beams must
    equal those of a fresh decode finalized separately."""
    cat = synth.catalog(100_000, 4, ("zipf",) * 4, [70, 1])
    trie = Trie(cat, device="cuda")
    S = 1400                                           # W1's released range + the tail hold W3
    beams = Beams(trie, S, 8, 512)
    out = beams.set_finish_outputs(True)
    live, got = {}, {}                                 # key -> [req id, base, width, steps]

    def admit(ws):
        ids, bases = beams.init(np.asarray([w for _, w in ws], dtype=np.int32))
        for (key, w), rid, base in zip(ws, ids, bases):
            live[key] = [int(rid), int(base), w, 0]

    def step():
        host = np.zeros((S, 256), dtype=np.float32)
        for key, (rid, base, w, t) in live.items():
            host[base:base + w] = synth.logits_rowkeyed(70, t, key, w, 2.0)
        beams.step(torch.from_numpy(host).cuda())
        torch.cuda.synchronize()
        for key in list(live):
            v = live[key]
            v[3] += 1
            if v[3] == 4:                               # finished by this step: read its row now
                rid = v[0]
                c = int(out["counts"][rid].item())
                got[key] = {"counts": c, "sids": out["sids"][rid, :c].cpu().numpy(),
                            "scores": out["scores"][rid, :c].cpu().numpy(),
                            "items": out["items"][rid, :c].cpu().numpy()}
                assert (out["items"][rid, c:] == -1).all().item()
                del live[key]

    W1, W2, W3 = [(1, 300), (2, 64)], [(3, 128), (4, 7), (5, 200)], [(6, 250), (7, 50), (8, 512)]
    admit(W1)
    step(); step()
    admit(W2)
    step(); step()                                      # W1 finishes and is released
    assert beams.status()["free_slots"] == S - 335
    admit(W3)                                           # reuses W1's slots and ids
    step(); step()                                      # W2 finishes
    step(); step()                                      # W3 finishes
    beams.check()
    assert not live and beams.status()["free_slots"] == S
    for ws in (W1, W2, W3):
        widths = [w for _, w in ws]
        ref = _decode(trie, widths, lambda t, i, w, ws=ws: synth.logits_rowkeyed(70, t, ws[i][0], w, 2.0), False)
        for i, (key, _) in enumerate(ws):
            c = int(ref["counts"][i])
            assert got[key]["counts"] == c, key
            for k in ("sids", "scores", "items"):
                assert np.array_equal(got[key][k], ref[k][i][:c]), (key, k)


def test_finish_mode_off_again():
    """Turning the mode off restores the separate finalize."""
    trie = Trie(synth.catalog(30_000, 3, ("zipf",) * 3, [71, 1]), device="cuda")
    beams = Beams(trie, 100, 2, 64)
    beams.set_finish_outputs(True)
    beams.set_finish_outputs(None)
    ids, bases = beams.init(np.asarray([64, 30], dtype=np.int32))
    for t in range(3):
        host = np.zeros((100, 256), dtype=np.float32)
        for i, (w, b) in enumerate(zip([64, 30], bases)):
            host[b:b + w] = synth.logits_rowkeyed(71, t, i, w, 2.0)
        beams.step(torch.from_numpy(host).cuda())
    assert beams.status()["finished"] == 2
    out = beams.finalize(ids)
    assert list(out["counts"]) == [64, 30]


def test_finish_under_timing_relaunches():
    """With kernel timing on, each kernel of a step is launched several times back to back;
    the finishing step frees the record it reads, which must keep the input's row count so
    that every relaunch computes the same beams. Catalogs where the last step has fewer
    input rows than beams (3 and 100 rows -> 512 beams) tell the two counts apart: the
    first merges inside the tile kernel, the second in the merge kernel."""
    for n1, n2 in ((3, 300), (100, 10)):
        a, b = np.meshgrid(np.arange(n1), np.arange(n2), indexing="ij")
        trie = Trie(np.stack([a.ravel(), b.ravel()], axis=1).astype(np.uint8), device="cuda")
        fn = _rowkeyed(72)
        res = []
        for repeat in (0, 3):
            beams = Beams(trie, 600, 2, 512)
            out = beams.set_finish_outputs(True)
            if repeat:
                beams.enable_timing(2, repeat)
            ids, bases = beams.init(np.asarray([512, 40], dtype=np.int32))
            for t in range(2):
                host = np.zeros((600, 256), dtype=np.float32)
                for i, (w, base) in enumerate(zip([512, 40], bases)):
                    host[base:base + w] = fn(t, i, w)
                beams.step(torch.from_numpy(host).cuda())
            torch.cuda.synchronize()
            res.append({k: v.cpu().numpy()[np.asarray(ids)] for k, v in out.items()})
            beams.check()
        _same(res[0], res[1])
        assert int(res[0]["counts"][0]) == 512


def _decode_exports(trie, widths, logits_fn, export_each, norm="children", temperature=0.0, bf16=False,
                    repeat=0):
    """A decode finalized at the end. Back-to-back steps leave each step's merge to the next
    step's tile kernel; an export after every step (export_each) makes every merge run in
    the merge kernel instead. Returns the finalize result and the state after every step."""
    S = int(sum(widths))
    beams = Beams(trie, S, len(widths), max(widths), norm=norm)
    if repeat:
        beams.enable_timing(trie.L, repeat)
    ids, bases = beams.init(np.asarray(widths, dtype=np.int32))
    states = []
    for t in range(trie.L):
        host = np.zeros((S, 256), dtype=np.float32)
        for i, (w, b) in enumerate(zip(widths, bases)):
            host[b:b + w] = logits_fn(t, i, w)
        x = torch.from_numpy(host).cuda()
        beams.step(x.to(torch.bfloat16) if bf16 else x, temperature=temperature, seed=1000 + t)
        if export_each:
            states.append({k: v.cpu().numpy() for k, v in beams.export().items()})
    if not export_each:
        states.append({k: v.cpu().numpy() for k, v in beams.export().items()})
    res = beams.finalize(ids)
    beams.check()
    return res, states


@pytest.mark.parametrize("name", sorted(CASES))
def test_deferred_merge_matches_merge_kernel(name):
    """Each step's merge done by the next step's tile kernel (every tile of a request
    merging it and keeping its own 64 rows) against the merge kernel: the final beams and
    the final state (rows, keys, nodes, back-pointers) must be bitwise equal."""
    cat_args, widths, seed, norm, temp, bf16 = CASES[name]
    trie = Trie(synth.catalog(*cat_args), device="cuda")
    fn = _rowkeyed(seed)
    a, sa = _decode_exports(trie, widths, fn, False, norm=norm, temperature=temp, bf16=bf16)
    b, sb = _decode_exports(trie, widths, fn, True, norm=norm, temperature=temp, bf16=bf16)
    _same(a, b)
    fa, fb = sa[-1], sb[-1]
    assert np.array_equal(fa["rows"], fb["rows"]) and np.array_equal(fa["level"], fb["level"])
    # entries past a request's live rows hold whatever the workspace held: not compared
    for rid, base in enumerate(np.cumsum([0] + widths[:-1])):
        k = int(fa["rows"][rid])
        for key in ("node", "score", "phi", "parent_slot"):
            assert np.array_equal(fa[key][base:base + k], fb[key][base:base + k]), (rid, key)
        assert np.array_equal(fa["hist"][-1, base:base + k], fb["hist"][-1, base:base + k]), rid
    if name == "merge_kernel_onchip_walk":
        c, _ = _decode_exports(trie, widths, fn, False, repeat=3)   # relaunched kernels: the same beams
        _same(a, c)


def test_deferred_merge_under_exact_ties():
    a_, b_, c_ = np.meshgrid(np.arange(256), np.arange(256), np.arange(4), indexing="ij")
    trie = Trie(np.stack([a_.ravel(), b_.ravel(), c_.ravel()], axis=1).astype(np.uint8), device="cuda")
    zero = lambda t, i, w: np.zeros((w, 256), dtype=np.float32)
    a, _ = _decode_exports(trie, [300, 64, 7], zero, False)
    b, _ = _decode_exports(trie, [300, 64, 7], zero, True)
    _same(a, b)


@pytest.mark.parametrize("mode", ["dense", "gather"])
def test_deferred_merge_lmhead(mode):
    """lm_head steps back to back (the dense head computes every row the request can have
    while the merge is pending; the children-only head runs in the tile kernel after the
    merge it does first) against an export after every step: bitwise equal beams and
    state."""
    cat = synth.catalog(60_000, 3, ("zipf",) * 3, [73, 1])
    trie = Trie(cat, device="cuda")
    widths, H = [512, 100, 20], 256
    S, R, B = sum(widths), len(widths), max(widths)
    w_dev = torch.from_numpy(np.stack([synth.lmhead_weight(73, lv, 256, H) for lv in range(3)]).view(np.int16))
    w_dev = w_dev.cuda().view(torch.bfloat16)
    hidden = [torch.from_numpy(synth.hidden_states(73, t, S, H).view(np.int16)).cuda().view(torch.bfloat16)
              for t in range(3)]
    res = []
    for export_each in (False, True):
        beams = Beams(trie, S, R, B)
        beams.set_read_mode(mode)
        ids, _ = beams.init(np.asarray(widths, dtype=np.int32))
        for t in range(3):
            beams.step_lmhead(hidden[t], w_dev)
            if export_each:
                beams.export()
        st = {k: v.cpu().numpy() for k, v in beams.export().items()}
        res.append((beams.finalize(ids), st))
        beams.check()
    _same(res[0][0], res[1][0])
    for rid, base in enumerate(np.cumsum([0] + widths[:-1])):
        k = int(res[0][1]["rows"][rid])
        assert k == int(res[1][1]["rows"][rid])
        assert np.array_equal(res[0][1]["hist"][-1, base:base + k], res[1][1]["hist"][-1, base:base + k]), rid


def test_deferred_merge_with_second_launch_chunk():
    """More request ids than one launch's arguments hold (400): the step is launched in
    chunks. 400 requests of width 128 step back to back (each merge left to the next
    step's tile kernel); then one more request is admitted, alone in the second chunk with
    one row. Its first step runs in the kernel that does the pending merges, which leaves
    its candidates to a merge like everyone else's. The beams and the final state must
    equal those of the same decode with an export (hence the merge kernel) after every
    step."""
    cat = synth.catalog(100_000, 4, ("zipf",) * 4, [74, 1])
    trie = Trie(cat, device="cuda")
    n0, w = 400, 128
    S = (n0 + 1) * w

    def run(export_each):
        beams = Beams(trie, S, n0 + 1, w)
        ids, bases = beams.init(np.full(n0, w, dtype=np.int32))
        ids, bases = list(ids), list(bases)
        level = [0] * n0
        for t in range(6):
            if t == 2:
                nid, nb = beams.init(np.asarray([w], dtype=np.int32))
                assert int(nid[0]) == n0
                ids.append(int(nid[0]))
                bases.append(int(nb[0]))
                level.append(0)
            host = np.zeros((S, 256), dtype=np.float32)
            for i, (b, lv) in enumerate(zip(bases, level)):
                if lv < 4:
                    host[b:b + w] = synth.logits_rowkeyed(74, lv, i, w, 2.0)
            beams.step(torch.from_numpy(host).cuda())
            level = [lv + 1 if lv < 4 else lv for lv in level]
            if export_each:
                beams.export()
            if t == 3:                                  # the first 400 are at depth 4
                first = beams.finalize(ids[:n0])
            if t == 5:
                last = beams.finalize(ids[n0:])
        beams.check()
        return first, last

    a1, a2 = run(False)
    b1, b2 = run(True)
    _same(a1, b1)
    _same(a2, b2)
    assert int(a2["counts"][0]) == w


def test_flush_between_steps_matches_export():
    """flush() (an export with every buffer NULL) after each step runs the step's merge on its
    own, copying nothing: the beams equal those of a decode that exports after every step."""
    cat = synth.catalog(100_000, 4, ("zipf",) * 4, [74, 1])
    trie = Trie(cat, device="cuda")
    widths = [512, 130, 64]
    fn = _rowkeyed(74)
    res = []
    for mode in ("flush", "export"):
        S = sum(widths)
        beams = Beams(trie, S, len(widths), max(widths))
        ids, bases = beams.init(np.asarray(widths, dtype=np.int32))
        for t in range(trie.L):
            host = np.zeros((S, 256), dtype=np.float32)
            for i, (w, b) in enumerate(zip(widths, bases)):
                host[b:b + w] = fn(t, i, w)
            beams.step(torch.from_numpy(host).cuda())
            if mode == "flush":
                beams.flush()
            else:
                beams.export()
        res.append(beams.finalize(ids))
        beams.check()
    _same(res[0], res[1])
