"""HIP path vs the oracle on the same seeded inputs (teacher-forced, every step).

Sizes span several 32-row tiles and ragged tails; edge cases cover width 1, widths
above the candidate count, single-child chains, exact ties, V < 256, L = 1 and the
normaliser flag. The full-size workloads are checked on sampled requests in
test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

import bruteforce as bf
import gpu_harness as gh
import oracle
from trie_constrained_beam_amd import Beams, TcbError, Trie, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    print(f"\n[gpu] {request.node.name}", flush=True)


CASES = {
    # name: (catalog args, widths, seed, sigma, bf16, mask_depths, norm)
    "uniform20k_l3_b50": ((20_000, 3, ("uniform",) * 3, [1, 1]), [50], 1, 2.0, False, None, "children"),
    "zipf100k_l4_b128x5": ((100_000, 4, ("zipf",) * 4, [31, 1]), [128] * 5, 31, 2.0, False, None, "children"),
    "zipf200k_l4_b512x3_bf16": ((200_000, 4, ("zipf",) * 4, [32, 1]), [512] * 3, 32, 3.0, True, None, "children"),
    "mixed_l5": ((300_000, 5, ("uniform",) + ("zipf",) * 4, [33, 1]), [50, 128, 256, 512, 1, 77, 300, 33],
                 33, 2.0, False, None, "children"),
    "level_norm": ((50_000, 4, ("zipf",) * 4, [34, 1]), [64] * 4 + [200], 34, 2.0, False, None, "level"),
    "csr_only": ((60_000, 4, ("zipf",) * 4, [35, 1]), [96, 512], 35, 2.0, False, 0, "children"),
    "mask_all_depths": ((60_000, 4, ("zipf",) * 4, [35, 1]), [96, 512], 35, 2.0, False, 4, "children"),
    "bf16_level": ((40_000, 3, ("uniform", "zipf", "zipf"), [36, 1]), [256, 45], 36, 3.0, True, None, "level"),
    # every request at most 64 rows: every step merged inside the tile kernel
    "zipf100k_l4_w64_in_tile": ((100_000, 4, ("zipf",) * 4, [37, 1]), [64, 1, 33, 50, 17, 64, 8], 37, 3.0, True,
                                None, "children"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_step_parity(name):
    cat_args, widths, seed, sigma, bf16, md, norm = CASES[name]
    cat = synth.catalog(*cat_args)
    run, stats = gh.run_rowkeyed(cat, widths, seed, sigma, bf16=bf16, mask_depths=md, norm=norm)
    assert stats["checked"] == len(widths) * cat.shape[1]
    run.beams.check()


def _prefix_logits_fn(seed, V, sigma=2.0):
    return lambda d, prefix_packed: synth.logits_prefixkeyed(seed, d, prefix_packed, sigma, V=V)


def _free_run(run, seed, sigma=2.0):
    """Drive the GPU with prefix-keyed logits generated from the GPU's own prefixes."""
    for t in range(run.L):
        st = run.state()
        rows_list = []
        for i, (rid, base) in enumerate(zip(run.ids, run.bases)):
            rows = int(st["rows"][rid])
            pref = gh.walk_prefixes(st["hist"], int(base), rows, t)
            x = synth.logits_prefixkeyed(seed, t, pref, sigma, V=256)
            rows_list.append(x)
        S = run.max_slots
        host = np.zeros((S, 256), dtype=np.float32)
        for x, base in zip(rows_list, run.bases):
            host[base:base + x.shape[0]] = x
        run.beams.step(torch.from_numpy(host).cuda())
    return run.beams.finalize(run.ids)


@pytest.mark.parametrize("case", range(40))
def test_tiny_catalogs_vs_bruteforce(case):
    """V in 2..5 (the unaligned load path), full enumeration replay as the reference."""
    rng = np.random.default_rng(500 + case)
    V = int(rng.integers(2, 6))
    L = int(rng.integers(1, 4))
    n = int(rng.integers(1, V ** L + 1))
    tuples = [tuple(int(c) for c in t) for t in np.ndindex(*(V,) * L)]
    cat = [tuples[i] for i in rng.choice(len(tuples), n, replace=False)]
    widths = [int(rng.integers(1, 9)) for _ in range(3)]
    norm = "children" if case % 3 else "level"
    seed = 900 + case
    run = gh.Run(np.asarray(cat, dtype=np.uint8), widths, V=V, norm=norm)

    for t in range(L):
        st = run.state()
        host = np.zeros((run.max_slots, V), dtype=np.float32)
        for rid, base in zip(run.ids, run.bases):
            rows = int(st["rows"][rid])
            pref = gh.walk_prefixes(st["hist"], int(base), rows, t)
            host[base:base + rows] = synth.logits_prefixkeyed(seed, t, pref, 2.0, V=V)
        run.beams.step(torch.from_numpy(host).cuda())
    out = run.beams.finalize(run.ids)

    def fn(d, p):
        key = 0
        for c in p:
            key = key * 256 + c
        return [float(v) for v in synth.logits_prefixkeyed(seed, d, [key], 2.0, V=V)[0]]
    catset = set(cat)
    for i, w in enumerate(widths):
        ref = bf.beam_replay(cat, V, w, fn, 0 if norm == "children" else 1)
        cnt = int(out["counts"][i])
        assert cnt == len(ref)
        got = [tuple(int(c) for c in out["sids"][i, j]) for j in range(cnt)]
        assert all(g in catset for g in got)
        ref_s = np.asarray([s for s, _ in ref])
        assert np.max(np.abs(out["scores"][i, :cnt] - ref_s)) < 1e-4
        # identical unless the replay has near-ties; with near-ties, everything clearly
        # above the last kept score must still be there
        gaps = np.abs(np.diff(ref_s)) if len(ref_s) > 1 else np.asarray([1.0])
        if gaps.min(initial=1.0) > 1e-5:
            assert got == [p for _, p in ref]
        else:
            clear = [p for s, p in ref if s > ref_s[-1] + 1e-5]
            assert set(clear) <= set(got)


def test_constant_logits_exact_ties():
    """All logits equal: every step is a tie broken by flat index; GPU == oracle exactly."""
    cat = synth.catalog(30_000, 4, ("zipf",) * 4, [40, 1])
    widths = [300, 64, 7]
    run = gh.Run(cat, widths)
    for t in range(4):
        rows = [np.zeros((w, 256), dtype=np.float32) for w in widths]
        post = run.step_and_check(t, rows, "f32")
    out = run.beams.finalize(run.ids)
    # closed form: a beam's score is -sum ln(fanout) along its path. Paths whose fanouts
    # come in a different order are equal in exact arithmetic but may round apart, so
    # only the per-step teacher-forced checks above compare tie order.
    kids = {}
    for sid in map(tuple, cat.tolist()):
        for d in range(4):
            kids.setdefault(sid[:d], set()).add(sid[d])
    for i, w in enumerate(widths):
        cnt = int(out["counts"][i])
        assert cnt == w
        for j in range(cnt):
            sid = tuple(int(c) for c in out["sids"][i, j])
            closed = -sum(np.log(len(kids[sid[:d]])) for d in range(4))
            assert abs(float(out["scores"][i, j]) - closed) < 1e-5


def test_exact_path_inside_merged_tile():
    """Requests of at most 64 rows merge inside the tile kernel. With every logit equal,
    64 rows x 256 children give 16384 exactly tied candidates, more than a tile keeps, so
    that tile takes its exact selection path and the merge then runs from memory in the
    same kernel: GPU == oracle, ties by flat index."""
    a, b, c = np.meshgrid(np.arange(256), np.arange(256), np.arange(4), indexing="ij")
    cat = np.stack([a.ravel(), b.ravel(), c.ravel()], axis=1).astype(np.uint8)   # complete to depth 2
    widths = [64, 17]
    run = gh.Run(cat, widths)
    for t in range(3):
        rows = [np.zeros((w, 256), dtype=np.float32) for w in widths]
        run.step_and_check(t, rows, "f32")
    out = run.beams.finalize(run.ids)
    for i, w in enumerate(widths):
        assert int(out["counts"][i]) == w


def test_single_child_chain_and_width_one():
    cat = np.array([[0, 5, 7, 1], [1, 2, 0, 0], [1, 2, 1, 0], [1, 2, 2, 0], [1, 3, 3, 3],
                    [2, 0, 0, 0]], dtype=np.uint8)
    for widths in ([1, 1], [16, 3], [2]):
        run = gh.Run(cat, widths)
        for t in range(4):
            run.step_and_check(t, gh.rowkeyed_logits(41, t, widths, 2.0, False), "f32")
        out = run.beams.finalize(run.ids)
        for i, w in enumerate(widths):
            assert int(out["counts"][i]) == min(w, 6)


def test_single_level_catalog():
    cat = np.arange(200, dtype=np.uint8).reshape(-1, 1)
    run = gh.Run(cat, [50, 256])
    run.step_and_check(0, gh.rowkeyed_logits(42, 0, [50, 256], 2.0, False), "f32")
    out = run.beams.finalize(run.ids)
    assert list(out["counts"]) == [50, 200]
    assert (out["items"][1, :200] == out["sids"][1, :200, 0]).all()


def test_mask_vs_csr_bitwise():
    """The dense-mask and CSR child paths give bit-identical states: randomized waves
    (catalog depth, size and code distributions, beam widths, logit scale and dtype, read
    mode) stepped side by side with every depth masked and with none, at least 10,000
    request-steps in all (the randomized dense-vs-sparse comparison of the SGLang
    deployment write-up, applied to the two child-set forms)."""
    rng = np.random.default_rng(43)
    request_steps = 0
    case = 0
    while request_steps < 10_000:
        L = int(rng.integers(3, 6))
        dists = tuple(str(x) for x in rng.choice(["uniform", "zipf"], L))
        n = int(rng.integers(20_000, 150_000))
        cat = synth.catalog(n, L, dists, [43, case])
        widths = [int(w) for w in rng.choice([1, 7, 33, 50, 64, 100, 128, 256, 512], int(rng.integers(100, 500)))]
        sigma = float(rng.choice([0.5, 2.0, 3.0]))
        bf16 = bool(rng.integers(0, 2))
        mode = str(rng.choice(["auto", "dense", "gather"]))
        runs = [gh.Run(cat, widths, mask_depths=md, max_slots=sum(widths), read_mode=mode) for md in (0, L)]
        for t in range(L):
            x = gh.rowkeyed_logits(43 + case, t, widths, sigma, bf16)
            host = np.zeros((sum(widths), 256), dtype=np.uint16 if bf16 else np.float32)
            for xi, base in zip(x, runs[0].bases):
                host[base:base + xi.shape[0]] = xi
            dev = torch.from_numpy(host.view(np.int16) if bf16 else host).cuda()
            states = []
            for r in runs:
                r.beams.step(dev.view(torch.bfloat16) if bf16 else dev)
                states.append(r.state())
            a, b = states
            assert np.array_equal(a["rows"], b["rows"]) and np.array_equal(a["level"], b["level"]), (case, t)
            # live rows and the level just written (the rest of the workspace is never read;
            # earlier levels were compared at their own step)
            for rid, base in zip(runs[0].ids, runs[0].bases):
                k = int(a["rows"][rid])
                sl = slice(int(base), int(base) + k)
                for key in ("node", "parent_slot"):
                    assert np.array_equal(a[key][sl], b[key][sl]), (case, t, rid, key)
                assert np.array_equal(a["score"][sl].view(np.uint32), b["score"][sl].view(np.uint32)), (case, t, rid)
                assert np.array_equal(a["hist"][t, sl], b["hist"][t, sl]), (case, t, rid)
            request_steps += len(widths)
        for r in runs:
            r.beams.check()
        print(f"case {case}: L={L} {dists} {n} SIDs, {len(widths)} requests, sigma {sigma}, "
              f"{'bf16' if bf16 else 'f32'}, {mode}; {request_steps} request-steps so far", flush=True)
        case += 1
    print(f"mask vs CSR: {request_steps} request-steps over {case} random waves", flush=True)


def test_determinism_bitwise():
    cat = synth.catalog(200_000, 4, ("zipf",) * 4, [44, 1])
    widths = [512] * 6 + [128] * 4
    outs = []
    for _ in range(2):
        run = gh.Run(cat, widths)
        for t in range(4):
            x = gh.rowkeyed_logits(44, t, widths, 3.0, True)
            host = np.zeros((run.max_slots, 256), dtype=np.uint16)
            for xi, base in zip(x, run.bases):
                host[base:base + xi.shape[0]] = xi
            run.beams.step(torch.from_numpy(host.view(np.int16)).cuda().view(torch.bfloat16))
        outs.append(run.beams.finalize(run.ids))
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[1][k]), k


def test_in_tile_merge_matches_merge_kernel():
    """Requests of at most 64 rows are merged inside the tile kernel when the whole launch
    has at most 64 rows per request; one wider request in the launch sends every request
    through k_merge. The narrow requests' rows, back-pointers and final SIDs must be bitwise
    the same either way (row-keyed logits give them the same inputs in both runs)."""
    cat = synth.catalog(100_000, 4, ("zipf",) * 4, [46, 1])
    narrow = [64, 33, 1, 50]
    res = []
    for widths in (narrow, narrow + [300]):
        run = gh.Run(cat, widths)
        states = []
        for t in range(4):
            x = gh.rowkeyed_logits(46, t, widths, 2.5, False)
            host = np.zeros((run.max_slots, 256), dtype=np.float32)
            for xi, base in zip(x, run.bases):
                host[base:base + xi.shape[0]] = xi
            run.beams.step(torch.from_numpy(host).cuda())
            ex = {k: v.cpu().numpy() for k, v in run.beams.export().items()}
            st = []
            for i, (rid, base) in enumerate(zip(run.ids[:len(narrow)], run.bases)):
                k = int(ex["rows"][rid])
                st.append((k, ex["node"][base:base + k].copy(), ex["score"][base:base + k].view(np.int32).copy(),
                           ex["hist"][t, base:base + k].copy()))
            states.append(st)
        fin = run.beams.finalize(run.ids)
        res.append((states, {k: v[:len(narrow)] for k, v in fin.items()}))
    for t in range(4):
        for i in range(len(narrow)):
            a, b = res[0][0][t][i], res[1][0][t][i]
            assert a[0] == b[0], (t, i)
            for u, v in zip(a[1:], b[1:]):
                assert np.array_equal(u, v), (t, i)
    fa, fb = res[0][1], res[1][1]
    assert np.array_equal(fa["counts"], fb["counts"])
    for i, c in enumerate(fa["counts"]):
        for k in fa:
            if k != "counts":
                assert np.array_equal(fa[k][i][:int(c)], fb[k][i][:int(c)]), (k, i)


def test_first_step_reads_no_initial_state():
    """A request's first step starts from its known initial state without reading it (the
    state is written only when something else reads it first). New requests admitted
    mid-decode beside older ones, and into slots that held other requests' rows, with no
    export in between, must decode bitwise as in a fresh wave."""
    cat = synth.catalog(100_000, 4, ("zipf",) * 4, [47, 1])
    trie = Trie(cat, device="cuda")
    S = 1200

    def run(plan):
        """plan: list of ("init", [(key, width), ...]) / ("step",) / ("fin", [key, ...])."""
        beams = Beams(trie, S, 8, 512)
        live, out = {}, {}                              # key -> [req id, base, width, steps taken]
        for op in plan:
            if op[0] == "init":
                ids, bases = beams.init(np.asarray([w for _, w in op[1]], dtype=np.int32))
                for (key, w), rid, base in zip(op[1], ids, bases):
                    live[key] = [int(rid), int(base), w, 0]
            elif op[0] == "step":
                host = np.zeros((S, 256), dtype=np.float32)
                for key, (rid, base, w, t) in live.items():
                    if t < 4:
                        host[base:base + w] = synth.logits_rowkeyed(47, t, key, w, 2.0)
                beams.step(torch.from_numpy(host).cuda())
                for v in live.values():
                    v[3] = min(v[3] + 1, 4)
            else:
                fin = beams.finalize(np.asarray([live[k][0] for k in op[1]], dtype=np.int32))
                for i, k in enumerate(op[1]):
                    c = int(fin["counts"][i])
                    out[k] = (c, fin["sids"][i][:c].copy(), fin["scores"][i][:c].copy(), fin["items"][i][:c].copy())
                    del live[k]
        return out

    W1, W2, W3 = [(1, 300), (2, 64)], [(3, 128), (4, 7), (5, 200)], [(6, 250), (7, 50)]
    mixed = run([("init", W1), ("step",), ("step",), ("init", W2), ("step",), ("step",), ("fin", [1, 2]),
                 ("init", W3), ("step",), ("step",), ("fin", [3, 4, 5]), ("step",), ("step",), ("fin", [6, 7])])
    fresh = {}
    for Wn in (W2, W3):
        fresh.update(run([("init", Wn), ("step",), ("step",), ("step",), ("step",), ("fin", [k for k, _ in Wn])]))
    for key in fresh:
        a, b = mixed[key], fresh[key]
        assert a[0] == b[0], key
        for u, v in zip(a[1:], b[1:]):
            assert np.array_equal(u, v), key


def test_finalize_legality_items_and_device_variant():
    cat = synth.catalog(80_000, 4, ("zipf",) * 4, [45, 1])
    cat = np.concatenate([cat, cat[:5000]])               # duplicates map to the lowest row
    widths = [256, 50, 512]
    outs = []
    for variant in ("host", "device"):
        run = gh.Run(cat, widths)
        for t in range(4):
            run.step_and_check(t, gh.rowkeyed_logits(45, t, widths, 2.0, False), "f32")
        if variant == "host":
            outs.append(run.beams.finalize(run.ids))
        else:
            d = run.beams.finalize_device(run.ids)
            torch.cuda.synchronize()
            outs.append({k: v.cpu().numpy() for k, v in d.items()})
        assert run.beams.status()["free_slots"] == run.max_slots
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[1][k]), k
    out = outs[0]
    keys = synth.pack_sids(cat)
    first = {}
    for row, key in enumerate(keys):
        first.setdefault(int(key), row)
    for i, w in enumerate(widths):
        cnt = int(out["counts"][i])
        assert cnt == w
        sk = synth.pack_sids(out["sids"][i, :cnt])
        assert len(set(sk.tolist())) == cnt                       # no duplicate SIDs
        for key, item in zip(sk, out["items"][i, :cnt]):
            assert first[int(key)] == int(item)                     # legal, lowest row
        assert (np.diff(out["scores"][i, :cnt]) <= 0).all()
        assert np.isneginf(out["scores"][i, cnt:]).all() and (out["items"][i, cnt:] == -1).all()


def test_nonfinite_logits_flagged():
    cat = synth.catalog(5000, 3, ("uniform",) * 3, [46, 1])
    trie = Trie(cat, device="cuda")
    b = Beams(trie, 64, 1, 64)
    b.set_validate(True)
    b.init([64])
    x = torch.zeros((64, 256), device="cuda")
    x[0, 17] = float("nan")
    b.step(x)
    with pytest.raises(TcbError, match="NONFINITE"):
        b.check()


def test_admission_between_steps_and_slot_reuse():
    """Requests join a running wave between steps, finish, and their slots are reused."""
    cat = synth.catalog(100_000, 3, ("uniform", "zipf", "zipf"), [47, 1])
    trie = Trie(cat, device="cuda")
    otrie = oracle.OracleTrie(cat)
    S = 1000
    b = Beams(trie, S, 8, 512)
    live = {}          # rid -> (base, width, seed index, level)
    rng = np.random.default_rng(47)
    admitted = 0
    for g in range(9):
        want = [int(w) for w in rng.choice([50, 128, 256, 512], 2)]
        st = b.status()
        take = []
        for w in want:
            if w <= st["free_slots"] - sum(take) and st["free_requests"] > len(take):
                take.append(w)
        if take:
            try:
                ids, bases = b.init(take)
            except TcbError:
                ids, bases = [], []          # fragmentation: admission is all or nothing
                take = []
            for rid, base, w in zip(ids, bases, take):
                live[int(rid)] = [int(base), w, admitted, 0]
                admitted += 1
        ex = {k: v.cpu().numpy() for k, v in b.export().items()}
        host = np.zeros((S, 256), dtype=np.float32)
        expect = {}
        for rid, (base, w, q, lv) in live.items():
            if lv >= 3:
                continue
            rows = int(ex["rows"][rid])
            x = synth.logits_rowkeyed(47, lv, q, w, 2.0)
            host[base:base + w] = x
            pref = gh.walk_prefixes(ex["hist"], base, rows, lv)
            expect[rid] = oracle.expand_request(otrie, lv, pref, ex["score"][base:base + rows].astype(np.float64),
                                                x[:rows].astype(np.float64), w)
        b.step(torch.from_numpy(host).cuda())
        post = {k: v.cpu().numpy() for k, v in b.export().items()}
        for rid, ref in expect.items():
            base, w, q, lv = live[rid]
            k = int(post["rows"][rid])
            h = post["hist"][lv, base:base + k].astype(np.int64)
            gh.compare_step(ref, h >> 8, h & 255, post["node"][base:base + k], post["score"][base:base + k],
                            ctx=f"rid {rid} level {lv}")
            live[rid][3] += 1
        done = [rid for rid, v in live.items() if v[3] >= 3]
        if done:
            out = b.finalize(done)
            assert all(int(c) > 0 for c in out["counts"])
            for rid in done:
                del live[rid]
    assert admitted >= 6
