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
