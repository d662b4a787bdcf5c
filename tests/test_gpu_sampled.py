"""Gumbel top-k without replacement above temperature 0, on the GPU, against the oracle.

Teacher-forced per step (the oracle starts every step from the GPU's own pre-step rows,
keys and log-probabilities), the kept set, order, keys and log-probabilities follow the
oracle's stochastic beam search up to float32 rounding; over many requests the returned
SIDs' inclusion frequencies match the exact Plackett-Luce probabilities; equal seeds
give identical results.
"""
import math

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


def _dev(host, bf16):
    if bf16:
        return torch.from_numpy(host.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(host).cuda()


def _sampled_run(cat, widths, seed, sigma, T, bf16=False, norm="children", mask_depths=None):
    run = gh.Run(cat, widths, norm=norm, mask_depths=mask_depths)
    dt = "bf16" if bf16 else "f32"
    stats = {}
    for t in range(run.L):
        xs = gh.rowkeyed_logits(seed, t, widths, sigma, bf16)
        host = np.zeros((run.max_slots, 256), dtype=np.uint16 if bf16 else np.float32)
        for x, b in zip(xs, run.bases):
            host[b:b + x.shape[0]] = x
        pre = run.state()
        run.beams.step(_dev(host, bf16), temperature=T, seed=1000 + t)
        post = run.state()
        for i, (rid, base) in enumerate(zip(run.ids, run.bases)):
            rid, base = int(rid), int(base)
            rows = int(pre["rows"][rid])
            pref = gh.walk_prefixes(pre["hist"], base, rows, t)
            ref = oracle.expand_request_sampled(
                run.otrie, t, pref, pre["phi"][base:base + rows].astype(np.float64),
                pre["score"][base:base + rows].astype(np.float64), oracle.widen_logits(xs[i][:rows], dt),
                widths[i], T, 1000 + t, rid, run.norm)
            k = int(post["rows"][rid])
            d = gh.compare_sampled_step(ref, post, base, k, t, ctx=f"req {i} step {t} T {T}")
            stats["near_ties"] = stats.get("near_ties", 0) + d["near_ties"]
            stats["checked"] = stats.get("checked", 0) + 1
    run.beams.check()
    return run, stats


@pytest.mark.parametrize("T", [1.0, 0.6, 2.5])
def test_sampled_step_parity_uniform(T):
    cat = synth.catalog(30_000, 4, ("uniform",) * 4, [71, 1])
    run, stats = _sampled_run(cat, [64, 130, 7, 512], 71, 2.0, T)
    assert stats["checked"] == 16


def test_sampled_step_parity_zipf_bf16():
    cat = synth.catalog(200_000, 4, ("zipf",) * 4, [72, 1])
    _sampled_run(cat, [512, 256, 50], 72, 3.0, 1.0, bf16=True)


def test_sampled_step_parity_level_norm_and_csr():
    cat = synth.catalog(20_000, 3, ("uniform",) * 3, [73, 1])
    _sampled_run(cat, [100, 33], 73, 2.0, 0.8, norm="level")
    _sampled_run(cat, [100, 33], 73, 2.0, 0.8, mask_depths=0)


def _decode(cat, widths, seeds, T, sigma=2.0):
    trie = Trie(cat, device="cuda")
    S = sum(widths)
    beams = Beams(trie, S, len(widths), max(widths))
    ids, bases = beams.init(widths)
    for t in range(cat.shape[1]):
        host = np.zeros((S, 256), dtype=np.float32)
        for i, (w, b) in enumerate(zip(widths, bases)):
            host[b:b + w] = synth.logits_rowkeyed(74, t, i, w, sigma)
        beams.step(torch.from_numpy(host).cuda(), temperature=T, seed=seeds[t])
    return beams.finalize(ids)


def test_sampled_decode_legal_deterministic():
    cat = synth.catalog(50_000, 4, ("zipf",) * 4, [74, 1])
    keys = synth.pack_sids(cat)
    catset = set(keys.tolist())
    widths = [256, 64, 512]
    a = _decode(cat, widths, [1, 2, 3, 4], 1.0)
    b = _decode(cat, widths, [1, 2, 3, 4], 1.0)
    c = _decode(cat, widths, [5, 6, 7, 8], 1.0)
    for k in ("sids", "scores", "items", "counts"):
        assert np.array_equal(a[k], b[k]), k                  # same seeds: identical
    assert not np.array_equal(a["sids"], c["sids"])            # other seeds: another sample
    for i, w in enumerate(widths):
        n = int(a["counts"][i])
        assert n == w
        got = synth.pack_sids(a["sids"][i, :n])
        assert np.unique(got).size == n and all(int(g) in catset for g in got)
        assert np.isfinite(a["scores"][i, :n]).all() and (a["scores"][i, :n] <= 0).all()


def test_sampled_inclusion_matches_plackett_luce():
    """256 requests per wave on one tiny trie: each request id draws its own noise, so
    every wave is 256 independent samples of k SIDs without replacement."""
    cat = np.asarray([(0, 0, 0)] + [(1, a, b) for a in range(3) for b in range(3)] + [(2, 0, 0), (2, 0, 1)],
                     dtype=np.uint8)
    V, k, T = 256, 3, 1.0
    base_logits = {(): [1.5, 0.0, 0.3], (1,): [0.0, 0.2, -0.3], (1, 0): [0.1, 0.0, -0.2],
                   (1, 1): [0.0, 0.4, 0.0], (1, 2): [0.3, 0.0, 0.0], (2, 0): [0.6, 0.0, 0.0]}
    fn = lambda d, p: base_logits.get(p, [0.0, 0.0, 0.0]) + [0.0] * (V - 3)
    incl = bf.pl_inclusion(bf.leaf_probs([tuple(c) for c in cat.tolist()], V, fn, T), k)
    trie = Trie(cat, device="cuda")
    n_req = 256
    beams = Beams(trie, n_req * k, n_req, k)
    counts = dict.fromkeys(incl, 0)
    n_samples = 0
    for wave in range(12):
        ids, bases = beams.init([k] * n_req)
        for t in range(3):
            pre = {kk: v.cpu().numpy() for kk, v in beams.export().items()}
            host = np.zeros((n_req * k, V), dtype=np.float32)
            for rid, base in zip(ids, bases):
                rows = int(pre["rows"][rid])
                pref = gh.walk_prefixes(pre["hist"], int(base), rows, t)
                for r in range(rows):
                    p = tuple((int(pref[r]) >> (8 * (t - 1 - j))) & 255 for j in range(t))
                    host[base + r] = fn(t, p)
            beams.step(torch.from_numpy(host).cuda(), temperature=T, seed=97 + 7 * wave + t)
        out = beams.finalize(ids)
        for i in range(n_req):
            for row in out["sids"][i, :int(out["counts"][i])]:
                counts[tuple(int(c) for c in row)] += 1
        n_samples += n_req
    z = max(abs(counts[s] / n_samples - q) / math.sqrt(q * (1 - q) / n_samples + 1e-12) for s, q in incl.items())
    assert z < 5.0, (z, {s: (counts[s] / n_samples, q) for s, q in incl.items()})


def test_sampled_argument_errors():
    cat = synth.catalog(2000, 2, ("uniform",) * 2, [75, 1])
    trie = Trie(cat, device="cuda")
    beams = Beams(trie, 64, 1, 64)
    beams.init([64])
    x = torch.zeros((64, 256), dtype=torch.float32, device="cuda")
    for bad in (-1.0, float("inf"), float("nan"), 1e-45):
        with pytest.raises(TcbError, match="ARG"):
            beams.step(x, temperature=bad, seed=1)
