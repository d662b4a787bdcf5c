"""Decoding without the SID constraint (open vocabulary) on the GPU, against the oracle,
and the invalid-rate comparison with the constrained decode.

flashrec 0.1.0, Evaluation: with the SID constraint no beam is illegal; engines without
it leave a share of their beams outside the catalog. Here both modes run the same
kernels on the same logits; the oracle's open mode is pinned against torch's plain
beam search.
"""
import numpy as np
import pytest
import torch

import gpu_harness as gh
from trie_constrained_beam_amd import Beams, Trie, invalid_rate, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    print(f"\n[gpu] {request.node.name}", flush=True)


@pytest.mark.parametrize("bf16", [False, True])
def test_open_step_parity(bf16):
    """Every step teacher-forced against the oracle: all 256 codes are candidates, and a
    node is -1 exactly when the prefix has left the catalog."""
    cat = synth.catalog(20_000, 4, ("uniform",) * 4, [81, 1])
    run, stats = gh.run_rowkeyed(cat, [64, 300, 7, 512], 81, 2.0, bf16=bf16, norm="open")
    assert stats["checked"] == 16
    st = run.state()
    assert (st["node"][run.bases[3]:run.bases[3] + 512] == -1).any()   # some beams left the catalog


def test_open_sampled_step_parity():
    import test_gpu_sampled as ts
    cat = synth.catalog(20_000, 3, ("uniform",) * 3, [82, 1])
    ts._sampled_run(cat, [100, 256], 82, 2.0, 1.0, norm="open")


def _decode(cat, widths, norm, seed=83):
    trie = Trie(cat, device="cuda")
    S = sum(widths)
    beams = Beams(trie, S, len(widths), max(widths), norm=norm)
    ids, bases = beams.init(widths)
    for t in range(cat.shape[1]):
        host = np.zeros((S, 256), dtype=np.float32)
        for i, (w, b) in enumerate(zip(widths, bases)):
            host[b:b + w] = synth.logits_rowkeyed(seed, t, i, w, 2.0)
        beams.step(torch.from_numpy(host).cuda())
    beams.check()
    return beams.finalize(ids)


def test_invalid_rate_constrained_vs_open():
    """Same logits, same kernels: the constrained decode returns only catalog SIDs, the
    open one leaves a share outside (items -1), and every item it does return is right."""
    # dense enough (30k of the 65,536 code pairs) that random logits land in the catalog
    # often; with sparse catalogs nearly every open beam is illegal
    cat = synth.catalog(30_000, 2, ("uniform",) * 2, [84, 1])
    keys = synth.pack_sids(cat)
    first = {}
    for row, k in enumerate(keys.tolist()):
        first.setdefault(k, row)
    widths = [512] * 8
    con = _decode(cat, widths, "children")
    opn = _decode(cat, widths, "open")
    assert invalid_rate(con) == 0.0
    rate = invalid_rate(opn)
    assert 0.0 < rate < 1.0, rate
    for i in range(len(widths)):
        n = int(opn["counts"][i])
        got = synth.pack_sids(opn["sids"][i, :n])
        assert np.unique(got).size == n
        for k, item in zip(got.tolist(), opn["items"][i, :n].tolist()):
            assert item == first.get(k, -1)
        assert (np.diff(opn["scores"][i, :n]) <= 0).all()
