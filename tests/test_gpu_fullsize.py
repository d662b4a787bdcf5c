"""The benchmark workloads at full size, in the launch configuration bench.py times.

Every workload runs on the GPU exactly as benchmarked (one wave holding all requests,
or FIFO admission under the 32,768-slot budget for the mixed wave). Sampled requests
are checked at every step against the oracle, teacher-forced from the GPU's pre-step
state; every finalized beam of every request is checked for legality (a catalog SID,
no duplicates, ranked best-first, the lowest catalog row as its item).
"""
import numpy as np
import pytest
import torch

import gpu_harness as gh
import oracle
from trie_constrained_beam_amd import Beams, Trie, run_wave, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    print(f"\n[gpu] {request.node.name}", flush=True)


_CACHE = {}


def _workload(name):
    if name not in _CACHE:
        wl = synth.WORKLOADS[name]
        cat = wl.catalog()
        keys = synth.pack_sids(cat)
        first = {}
        order = np.argsort(keys, kind="stable")
        sk = keys[order]
        newk = np.ones(sk.size, dtype=bool)
        newk[1:] = sk[1:] != sk[:-1]
        lowest = dict(zip(sk[newk].tolist(), order[newk].tolist()))
        _CACHE[name] = (wl, cat, oracle.OracleTrie(cat), lowest)
    return _CACHE[name]


def _check_legal(lowest, sids, scores, items, width, ctx):
    cnt = sids.shape[0]
    assert cnt <= width, ctx
    keys = synth.pack_sids(sids)
    assert np.unique(keys).size == cnt, f"{ctx}: duplicate SIDs"
    for key, item in zip(keys.tolist(), items.tolist()):
        assert lowest.get(key) == item, f"{ctx}: illegal SID or wrong item"
    assert (np.diff(scores) <= 0).all(), f"{ctx}: not ranked best-first"


def _check_request(run_state_pre, run_state_post, otrie, rid, base, level, x_rows, dtype, width, ctx, x64=None):
    rows = int(run_state_pre["rows"][rid])
    pref = gh.walk_prefixes(run_state_pre["hist"], base, rows, level)
    if x64 is None:
        x64 = oracle.widen_logits(x_rows[:rows], dtype)
    ref = oracle.expand_request(otrie, level, pref, run_state_pre["score"][base:base + rows].astype(np.float64),
                                x64, width)
    k = int(run_state_post["rows"][rid])
    h = run_state_post["hist"][level, base:base + k].astype(np.int64)
    gh.compare_step(ref, h >> 8, h & 255, run_state_post["node"][base:base + k],
                    run_state_post["score"][base:base + k], ctx=ctx)


def _state(beams):
    ex = beams.export()
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in ex.items()}


@pytest.mark.parametrize("name,sample", [
    ("b50x1_l3_20k_f32", [0]),
    ("b128x64_l4_1m_zipf_f32", [0, 17, 42, 63]),
    ("b512x32_l4_4m_zipf_bf16", list(range(32))),
])
def test_fullsize_one_wave(name, sample):
    wl, cat, otrie, lowest = _workload(name)
    widths = list(wl.widths)
    S, R, B = sum(widths), len(widths), max(widths)
    trie = Trie(cat, device="cuda")
    beams = Beams(trie, S, R, B)
    ids, bases = beams.init(widths)
    dt = "bf16" if wl.bf16 else "f32"
    for t in range(wl.L):
        xs = [synth.logits_rowkeyed(wl.seed, t, i, w, wl.sigma, bf16=wl.bf16) for i, w in enumerate(widths)]
        host = np.zeros((S, 256), dtype=np.uint16 if wl.bf16 else np.float32)
        for x, b in zip(xs, bases):
            host[b:b + x.shape[0]] = x
        dev = torch.from_numpy(host.view(np.int16) if wl.bf16 else host).cuda()
        pre = _state(beams)
        beams.step(dev.view(torch.bfloat16) if wl.bf16 else dev)
        post = _state(beams)
        for i in sample:
            _check_request(pre, post, otrie, int(ids[i]), int(bases[i]), t, xs[i], dt, widths[i],
                           f"{name} req {i} step {t}")
    beams.check()
    out = beams.finalize(ids)
    for i, w in enumerate(widths):
        c = int(out["counts"][i])
        assert c == w
        _check_legal(lowest, out["sids"][i, :c], out["scores"][i, :c], out["items"][i, :c], w, f"{name} req {i}")


def _capture(decode, n):
    """decode(c) for c < n, each captured as a HIP graph on a side stream, as bench.py
    captures its groups of decodes."""
    graphs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in range(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                decode(c)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return graphs


def test_fullsize_timed_route_graph_replay():
    """The route bench.py times, at its size: 32 requests x 512 beams, 4M Zipf catalog, bf16
    logits, steps back to back (each step's merge left to the next step's tile kernel), the
    last step writing every request's beams to the finish outputs, two decodes (of two input
    copies) captured per HIP graph and replayed. Every replay's outputs must equal, bitwise, a
    decode of the same inputs with an export after every step (each merge in the merge kernel,
    finalized separately), which test_fullsize_one_wave checks against the oracle step by step for all
    32 requests; the replays' beams must also be legal. Between replays the outputs are
    overwritten by eager work, so each replay must write all of them again."""
    wl, cat, otrie, lowest = _workload("b512x32_l4_4m_zipf_bf16")
    widths = list(wl.widths)
    S, R, B, L = sum(widths), len(widths), max(widths), wl.L
    trie = Trie(cat, device="cuda")
    bases = np.cumsum([0] + widths[:-1])
    host = []
    for t in range(L):
        h = np.zeros((S, 256), dtype=np.uint16)
        for i, (w, b) in enumerate(zip(widths, bases)):
            h[b:b + w] = synth.logits_rowkeyed(wl.seed, t, i, w, wl.sigma, bf16=True)
        host.append(h)
    pool = [[torch.from_numpy(h.view(np.int16)).cuda().view(torch.bfloat16) for h in host] for _ in range(2)]

    ref_beams = Beams(trie, S, R, B)
    ids, got_bases = ref_beams.init(widths)
    assert list(got_bases) == list(bases)
    for t in range(L):
        ref_beams.step(pool[0][t])
        ref_beams.export()
    ref = ref_beams.finalize(ids)
    ref_beams.check()

    beams = Beams(trie, S, R, B)
    out = beams.set_finish_outputs(True)

    def decode(c):
        rid, _ = beams.init(widths)
        assert list(rid) == list(ids)
        for t in range(L):
            beams.step(pool[c][t])
    decode(0)                                          # one eager decode, as the bench's warm-up
    torch.cuda.synchronize()
    graphs = _capture(lambda c: [decode(c), decode(1 - c)], 2)   # two decodes per graph
    idx = np.asarray(ids)
    for rep in range(4):
        out["sids"].fill_(0xAB)
        out["scores"].fill_(12345.0)
        out["items"].fill_(-7)
        out["counts"].fill_(-7)
        torch.cuda.synchronize()
        graphs[rep % 2].replay()
        torch.cuda.synchronize()
        got = {k: v.cpu().numpy()[idx] for k, v in out.items()}
        for k in ("counts", "sids", "scores", "items"):
            assert np.array_equal(got[k], ref[k]), (rep, k)
        if rep == 0:
            for i, w in enumerate(widths):
                c = int(got["counts"][i])
                assert c == w
                _check_legal(lowest, got["sids"][i, :c], got["scores"][i, :c], got["items"][i, :c], w,
                             f"replay req {i}")
    beams.check()


def test_fullsize_lmhead_route_graph_replay():
    """The lm_head workload as bench.py times it with the automatic head choice: 8 requests x
    512 beams, hidden 2048, 1M catalog; the dense MFMA head at levels 0-2 and the children's
    logits computed in the tile kernel at level 3, steps back to back (each merge in the next
    step's tile kernel, ahead of the in-tile head), finish outputs, two decodes per captured
    HIP graph. Every replay's outputs must equal, bitwise, a decode of the same inputs with an
    export after every step (test_fullsize_lmhead checks that route against the oracle), and
    the beams must be legal."""
    wl, cat, otrie, lowest = _workload("lmhead_b512x8_l4_1m_h2048")
    widths = list(wl.widths)
    S, R, B, L, H = sum(widths), len(widths), max(widths), wl.L, wl.hidden
    trie = Trie(cat, device="cuda")
    weights = np.stack([synth.lmhead_weight(wl.seed, lv, 256, H) for lv in range(L)])
    w_dev = torch.from_numpy(weights.view(np.int16)).cuda().view(torch.bfloat16)
    hid = [synth.hidden_states(wl.seed, t, S, H) for t in range(L)]
    pool = [[torch.from_numpy(h.view(np.int16)).cuda().view(torch.bfloat16) for h in hid] for _ in range(2)]

    ref_beams = Beams(trie, S, R, B)
    ref_beams.set_read_mode("auto")
    ids, _ = ref_beams.init(widths)
    for t in range(L):
        ref_beams.step_lmhead(pool[0][t], w_dev)
        ref_beams.export()
    ref = ref_beams.finalize(ids)
    ref_beams.check()

    beams = Beams(trie, S, R, B)
    beams.set_read_mode("auto")
    out = beams.set_finish_outputs(True)

    def decode(c):
        rid, _ = beams.init(widths)
        assert list(rid) == list(ids)
        for t in range(L):
            beams.step_lmhead(pool[c][t], w_dev)
    decode(0)
    torch.cuda.synchronize()
    graphs = _capture(lambda c: [decode(c), decode(1 - c)], 2)
    idx = np.asarray(ids)
    for rep in range(3):
        out["sids"].fill_(0xAB)
        out["scores"].fill_(12345.0)
        out["items"].fill_(-7)
        out["counts"].fill_(-7)
        torch.cuda.synchronize()
        graphs[rep % 2].replay()
        torch.cuda.synchronize()
        got = {k: v.cpu().numpy()[idx] for k, v in out.items()}
        for k in ("counts", "sids", "scores", "items"):
            assert np.array_equal(got[k], ref[k]), (rep, k)
        if rep == 0:
            for i, w in enumerate(widths):
                c = int(got["counts"][i])
                assert c == w
                _check_legal(lowest, got["sids"][i, :c], got["scores"][i, :c], got["items"][i, :c], w,
                             f"lm_head replay req {i}")
    beams.check()


def test_fullsize_mixed_wave_fifo():
    """256 requests, widths from {50, 128, 256, 512}, FIFO admission under 32,768 slots, L=5."""
    wl, cat, otrie, lowest = _workload("mixed256_l5_8m_f32")
    widths = list(wl.widths)
    trie = Trie(cat, device="cuda")
    beams = Beams(trie, wl.slot_budget, len(widths), max(widths))
    sample = set(range(0, len(widths), 16))
    checked = []
    live_widths = []

    def step_fn(step, live):
        live_widths.append(sum(q.width for q in live))
        host = np.zeros((wl.slot_budget, 256), dtype=np.float32)
        xs = {}
        for q in live:
            x = synth.logits_rowkeyed(wl.seed, q.level, q.index, q.width, wl.sigma)
            host[q.base:q.base + q.width] = x
            xs[q.index] = x
        pre = _state(beams)
        beams.step(torch.from_numpy(host).cuda())
        post = _state(beams)
        for q in live:
            if q.index in sample:
                _check_request(pre, post, otrie, q.rid, q.base, q.level, xs[q.index], "f32", q.width,
                               f"mixed req {q.index} level {q.level}")
                checked.append((q.index, q.level))

    results = run_wave(beams, widths, step_fn)
    assert sorted(results) == list(range(len(widths)))
    assert max(live_widths) <= wl.slot_budget
    assert len(checked) == len(sample) * wl.L
    for i, r in results.items():
        _check_legal(lowest, r["sids"], r["scores"], r["items"], widths[i], f"mixed req {i}")
    beams.check()


def test_fullsize_lmhead():
    """8 requests x 512 beams, hidden 2048, SID-range lm_head on MFMA, then the step."""
    wl, cat, otrie, lowest = _workload("lmhead_b512x8_l4_1m_h2048")
    widths = list(wl.widths)
    S, R, B, H = sum(widths), len(widths), max(widths), wl.hidden
    trie = Trie(cat, device="cuda")
    beams = Beams(trie, S, R, B)
    ids, bases = beams.init(widths)
    weights = np.stack([synth.lmhead_weight(wl.seed, lv, 256, H) for lv in range(wl.L)])
    w_dev = torch.from_numpy(weights.view(np.int16)).cuda().view(torch.bfloat16)
    for t in range(wl.L):
        hid = synth.hidden_states(wl.seed, t, S, H)
        pre = _state(beams)
        beams.step_lmhead(torch.from_numpy(hid.view(np.int16)).cuda().view(torch.bfloat16), w_dev)
        post = _state(beams)
        for i in (0, 5):
            base, rows = int(bases[i]), int(pre["rows"][ids[i]])
            x64 = oracle.lmhead_logits(hid[base:base + rows], weights[t])
            _check_request(pre, post, otrie, int(ids[i]), base, t, None, None, widths[i],
                           f"lmhead req {i} step {t}", x64=x64)
    beams.check()
    out = beams.finalize(ids)
    for i, w in enumerate(widths):
        c = int(out["counts"][i])
        _check_legal(lowest, out["sids"][i, :c], out["scores"][i, :c], out["items"][i, :c], w, f"lmhead req {i}")


def test_maximum_width():
    """Beam width 4096 (the largest accepted): the tiles' sample bound cannot prune and
    both kernels take their exact selection paths."""
    cat = synth.catalog(100_000, 3, ("uniform",) * 3, [61, 1])
    run, stats = gh.run_rowkeyed(cat, [4096, 1000], 61, 2.0)
    assert stats["checked"] == 6
