"""SID-range lm_head on the GPU (MFMA) followed by the constrained step, vs the oracle.

The oracle computes X = H W^T in float64 from the same bfloat16 hidden states and
weights (products of bf16 values are exact in float64), then takes the same masked
log-softmax / per-request top-n step. Teacher-forced: every step starts the oracle from
the GPU's own pre-step state.
"""
import numpy as np
import pytest
import torch

import gpu_harness as gh
import oracle
from trie_constrained_beam_amd import Beams, TcbError, Trie, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    print(f"\n[gpu] {request.node.name}", flush=True)


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _run_lmhead(cat, widths, H, seed, check_reqs=None, read_mode="auto"):
    run = gh.Run(cat, widths, read_mode=read_mode)
    L, S = run.L, run.max_slots
    weights = np.stack([synth.lmhead_weight(seed, lv, 256, H) for lv in range(L)])   # [L][256][H]
    w_dev = _bf16_dev(weights)
    stats = {}
    for t in range(L):
        hid = synth.hidden_states(seed, t, S, H)                                       # [S][H] by slot
        pre = run.state()
        run.beams.step_lmhead(_bf16_dev(hid), w_dev)
        post = run.state()
        for i in (range(len(widths)) if check_reqs is None else check_reqs):
            rid, base = int(run.ids[i]), int(run.bases[i])
            rows = int(pre["rows"][rid])
            pref = gh.walk_prefixes(pre["hist"], base, rows, t)
            x64 = oracle.lmhead_logits(hid[base:base + rows], weights[t])
            ref = oracle.expand_request(run.otrie, t, pref, pre["score"][base:base + rows].astype(np.float64),
                                        x64, widths[i])
            k = int(post["rows"][rid])
            h = post["hist"][t, base:base + k].astype(np.int64)
            d = gh.compare_step(ref, h >> 8, h & 255, post["node"][base:base + k], post["score"][base:base + k],
                                ctx=f"lm_head req {i} step {t}")
            stats["near_ties"] = stats.get("near_ties", 0) + d["near_ties"]
    run.beams.check()
    return run, stats


def test_lmhead_step_parity_small():
    cat = synth.catalog(30_000, 4, ("uniform",) * 4, [51, 1])
    _run_lmhead(cat, [64, 130, 7], 384, 51)


def test_lmhead_step_parity_wide_k():
    """K = 2048 (32 chunks of 64), several row tiles per request and a ragged tail."""
    cat = synth.catalog(60_000, 4, ("uniform",) * 4, [52, 1])
    _run_lmhead(cat, [512, 200], 2048, 52)


@pytest.mark.parametrize("H", [384, 1024])
def test_lmhead_narrow_beams_16_row_tiles(H):
    """Every request at most 16 beams wide: every level after the first runs the head on
    16-row tiles, with the generic K loop (H = 384) and the two-step loads (1024); the first
    step runs the one-row kernel."""
    cat = synth.catalog(20_000, 4, ("uniform",) * 4, [55, 1])
    _run_lmhead(cat, [16, 5, 9, 1], H, 55)


def test_lmhead_generic_k_every_tile_height():
    """H = 384 (the generic K loop, one K-step per load) with 8 requests of width 512 and the
    dense head at every level: on the 256-CU MI355X the first step runs the one-row kernel
    (48 pieces per row: a partial round of lanes), level 1 (2,048 rows) 32-row tiles and
    levels 2-3 64-row tiles; three requests checked against the oracle at every step."""
    cat = synth.catalog(300_000, 4, ("uniform",) * 4, [56, 1])
    _run_lmhead(cat, [512] * 8, 384, 56, check_reqs=[0, 3, 7], read_mode="dense")


def test_lmhead_matches_stepping_with_torch_logits():
    """The lm_head step equals tcb_beam_step on logits from an fp32 torch matmul of the same
    inputs up to fp32 rounding: same survivors wherever no near-tie decides."""
    cat = synth.catalog(20_000, 3, ("uniform",) * 3, [53, 1])
    widths = [100, 33]
    H = 512
    a = gh.Run(cat, widths)
    b = gh.Run(cat, widths)
    weights = np.stack([synth.lmhead_weight(53, lv, 256, H) for lv in range(3)])
    w_dev = _bf16_dev(weights)
    for t in range(3):
        hid = _bf16_dev(synth.hidden_states(53, t, a.max_slots, H))
        a.beams.step_lmhead(hid, w_dev)
        x = hid.float() @ w_dev[t].float().t().contiguous()
        b.beams.step(x.contiguous())
        sa, sb = a.state(), b.state()
        for i, rid in enumerate(a.ids):
            base, k = int(a.bases[i]), int(sa["rows"][rid])
            assert k == int(sb["rows"][rid])
            assert np.max(np.abs(sa["score"][base:base + k] - sb["score"][base:base + k])) < 1e-4


def test_lmhead_argument_errors():
    cat = synth.catalog(2000, 2, ("uniform",) * 2, [54, 1])
    trie = Trie(cat, device="cuda")
    beams = Beams(trie, 64, 1, 64)
    beams.init([64])
    w = torch.zeros((2, 256, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        beams.step_lmhead(torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda"), w[:1])
    with pytest.raises(TcbError, match="ARG"):
        beams.step_lmhead(torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda"), w[:, :, :64].contiguous())


@pytest.mark.parametrize("mode", ["dense", "gather"])
def test_lmhead_head_modes_parity(mode):
    """Dense head at every depth, or children-only pieces at every depth: both against the
    float64 oracle (the deep levels of this catalog have one or two children per row)."""
    cat = synth.catalog(40_000, 4, ("uniform",) * 4, [54, 1])
    _run_lmhead(cat, [256, 70, 9], 1024, 54, read_mode=mode)


def test_lmhead_children_only_wide_k_and_tail():
    """Children-only head with H = 4096 (8 chunks per lane) and rows past a tile boundary."""
    cat = synth.catalog(25_000, 3, ("zipf",) * 3, [55, 1])
    _run_lmhead(cat, [300, 5], 4096, 55, read_mode="gather")


def test_lmhead_children_only_deterministic():
    cat = synth.catalog(30_000, 4, ("uniform",) * 4, [56, 1])
    widths = [128, 64]
    H = 512
    weights = _bf16_dev(np.stack([synth.lmhead_weight(56, lv, 256, H) for lv in range(4)]))
    states = []
    for _ in range(2):
        run = gh.Run(cat, widths, read_mode="gather")
        for t in range(4):
            run.beams.step_lmhead(_bf16_dev(synth.hidden_states(56, t, run.max_slots, H)), weights)
        states.append(run.state())
    for k in ("node", "score", "hist", "rows"):
        a, b = states[0][k], states[1][k]
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b), k


def test_lmhead_dense_wide_k_deterministic():
    """Dense head with H = 4096 (32 K-steps per wave, two per load) against the oracle, then
    the same decode twice: bitwise equal states (the K split's partial sums are added in a
    fixed order)."""
    cat = synth.catalog(25_000, 3, ("zipf",) * 3, [57, 1])
    _run_lmhead(cat, [128, 33], 4096, 57, read_mode="dense")
    H = 4096
    weights = _bf16_dev(np.stack([synth.lmhead_weight(57, lv, 256, H) for lv in range(3)]))
    states = []
    for _ in range(2):
        run = gh.Run(cat, [128, 33], read_mode="dense")
        for t in range(3):
            run.beams.step_lmhead(_bf16_dev(synth.hidden_states(57, t, run.max_slots, H)), weights)
        states.append(run.state())
    for k in ("node", "score", "hist", "rows"):
        a, b = states[0][k], states[1][k]
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b), k


@pytest.mark.parametrize("H", [640, 2048, 4096])
def test_lmhead_in_tile_children_head_fused_route(H):
    """The automatic head choice on a uniform 4-level catalog: dense head at levels 0-2,
    and at level 3 (about one child per row) the children's logits computed inside the
    tile kernel, all 64 lanes of a wave on one (row, child) pair. H = 640: one round of
    loads in which lanes past the row's 80 pieces read and drop; H = 2048: one full round
    (256 pieces); H = 4096: two rounds. Checked against the oracle step by step (export after every
    step), then the same decode with the steps back to back (each merge done in the next
    step's tile kernel, so level 3's head runs after that merge, in the same kernel) must
    give bitwise the same finalized beams."""
    cat = synth.catalog(200_000, 4, ("uniform",) * 4, [58, 1])
    widths = [512, 512, 300, 9]
    run, _ = _run_lmhead(cat, widths, H, 58, check_reqs=[0, 2, 3], read_mode="auto")
    ref = run.beams.finalize(run.ids)
    L, S = run.L, run.max_slots
    w_dev = _bf16_dev(np.stack([synth.lmhead_weight(58, lv, 256, H) for lv in range(L)]))
    hidden = [_bf16_dev(synth.hidden_states(58, t, S, H)) for t in range(L)]
    beams = Beams(run.trie, S, len(widths), max(widths))
    beams.set_read_mode("auto")
    ids, _ = beams.init(np.asarray(widths, dtype=np.int32))
    for t in range(L):
        beams.step_lmhead(hidden[t], w_dev)
    got = beams.finalize(ids)
    beams.check()
    for k in ("counts", "sids", "scores", "items"):
        assert np.array_equal(got[k], ref[k]), k



def test_lmhead_mixed_levels_in_one_launch():
    """Requests admitted at different steps, so one lm_head launch holds requests at
    different levels: in the same tile kernel, rows at a dense depth read the dense head's
    logits while rows at the sparse last level get their children's logits computed in the
    tile (automatic choice), and a request admitted mid-decode takes its first step beside
    deeper ones (the MFMA head then computes its root row). First with an export around every
    step (so each merge runs as its own kernel), every request checked against the oracle at
    its own level; then the same schedule with the steps back to back (each merge done in the
    next step's tile kernel, before the in-tile head), whose finalized beams must be bitwise
    those of the checked run."""
    cat = synth.catalog(200_000, 4, ("uniform",) * 4, [59, 1])
    H, seed = 640, 59
    trie = Trie(cat, device="cuda")
    otrie = oracle.OracleTrie(cat.astype(np.int64))
    L, S = 4, 2048
    weights = np.stack([synth.lmhead_weight(seed, lv, 256, H) for lv in range(L)])
    w_dev = _bf16_dev(weights)
    admit = {0: [512, 100], 1: [256, 7], 2: [300]}           # step -> widths admitted before it
    hidden = [synth.hidden_states(seed, t, S, H) for t in range(L + 2)]

    def run(check):
        beams = Beams(trie, S, 8, 512)
        beams.set_read_mode("auto")
        live = []                                           # (req id, base, width, level)
        for t in range(L + 2):
            if t in admit:
                ids, bases = beams.init(np.asarray(admit[t], dtype=np.int32))
                live += [[int(r), int(b), w, 0] for r, b, w in zip(ids, bases, admit[t])]
            stepped = [q for q in live if q[3] < L]
            if not stepped:
                break
            pre = {k: v.cpu().numpy() for k, v in beams.export().items()} if check else None
            beams.step_lmhead(_bf16_dev(hidden[t]), w_dev)
            if check:
                post = {k: v.cpu().numpy() for k, v in beams.export().items()}
                for rid, base, w, lv in stepped:
                    assert int(pre["level"][rid]) == lv
                    rows = int(pre["rows"][rid])
                    pref = gh.walk_prefixes(pre["hist"], base, rows, lv)
                    x64 = oracle.lmhead_logits(hidden[t][base:base + rows], weights[lv])
                    ref = oracle.expand_request(otrie, lv, pref, pre["score"][base:base + rows].astype(np.float64),
                                                x64, w)
                    k = int(post["rows"][rid])
                    h = post["hist"][lv, base:base + k].astype(np.int64)
                    gh.compare_step(ref, h >> 8, h & 255, post["node"][base:base + k], post["score"][base:base + k],
                                    ctx=f"request {rid} level {lv} step {t}")
            for q in stepped:
                q[3] += 1
        res = beams.finalize(np.asarray([q[0] for q in live], dtype=np.int32))
        beams.check()
        return res

    checked = run(True)
    fused = run(False)
    for k in ("counts", "sids", "scores", "items"):
        assert np.array_equal(fused[k], checked[k]), k
