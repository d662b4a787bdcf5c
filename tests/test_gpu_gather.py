"""Sector-gathered logit reads: reading only the 16-byte pieces of a row that hold a
child must give bitwise the same beams as reading whole rows, and oracle parity."""
import numpy as np
import pytest
import torch

import gpu_harness as gh
from trie_constrained_beam_amd import synth

pytestmark = pytest.mark.gpu


def _pack(run, xs, bf16, ld=None):
    V = run.V
    ld = ld or V
    host = np.zeros((run.max_slots, ld), dtype=np.uint16 if bf16 else np.float32)
    for xi, base in zip(xs, run.bases):
        host[base:base + xi.shape[0], :V] = xi
    if bf16:
        dev = torch.from_numpy(host.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        dev = torch.from_numpy(host).cuda()
    return dev[:, :V]


def _bitwise(run, states_a, states_b, t, ctx):
    """Live rows of every request and the back-pointers this step wrote (the rest of the
    workspace is undefined; earlier steps' back-pointers were compared when written)."""
    assert np.array_equal(states_a["rows"], states_b["rows"]), ctx
    for rid, base in zip(run.ids, run.bases):
        rows = int(states_a["rows"][rid])
        sl = slice(int(base), int(base) + rows)
        for k in ("node", "score", "phi", "parent_slot"):
            a, b = states_a[k][sl], states_b[k][sl]
            if a.dtype == np.float32:
                a, b = a.view(np.uint32), b.view(np.uint32)
            assert np.array_equal(a, b), (ctx, k, int(rid))
        assert np.array_equal(states_a["hist"][t, sl], states_b["hist"][t, sl]), (ctx, "hist")


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("mask_depths", [None, 1])
def test_gather_vs_dense_bitwise(bf16, mask_depths):
    """Every read mode gives the same states, at every depth of a Zipf catalog (dense
    masks and CSR children, wide and narrow requests)."""
    rng = np.random.default_rng(71)
    cat = synth.catalog(150_000, 4, ("zipf",) * 4, [71, 1])
    widths = [int(w) for w in rng.choice([1, 9, 64, 200, 512], 120)]
    runs = [gh.Run(cat, widths, mask_depths=mask_depths, read_mode=m) for m in ("dense", "gather", "auto")]
    for t in range(4):
        dev = _pack(runs[0], gh.rowkeyed_logits(71, t, widths, 2.5, bf16), bf16)
        states = []
        for r in runs:
            r.beams.step(dev)
            states.append(r.state())
        _bitwise(runs[0], states[0], states[1], t, "gather")
        _bitwise(runs[0], states[0], states[2], t, "auto")


@pytest.mark.parametrize("bf16", [False, True])
def test_gather_parity(bf16):
    """Forced gathering against the oracle, on a sparse 4-level catalog."""
    cat = synth.catalog(60_000, 4, ("uniform", "zipf", "zipf", "zipf"), [72, 1])
    widths = [1, 5, 64, 130, 256, 512, 33]
    _, stats = gh.run_rowkeyed(cat, widths, 72, 2.0, bf16=bf16, read_mode="gather")
    assert stats["checked"] == len(widths) * 4


def test_gather_sampled_bitwise():
    """Sampled steps read the same values in both modes (keys and phi bitwise)."""
    cat = synth.catalog(80_000, 3, ("zipf",) * 3, [73, 1])
    widths = [4, 64, 300, 512]
    runs = [gh.Run(cat, widths, read_mode=m) for m in ("dense", "gather")]
    for t in range(3):
        dev = _pack(runs[0], gh.rowkeyed_logits(73, t, widths, 2.0, True), True)
        states = []
        for r in runs:
            r.beams.step(dev, temperature=0.8, seed=5)
            states.append(r.state())
        _bitwise(runs[0], states[0], states[1], t, "gather")


def test_gather_unaligned_rows_fall_back():
    """Rows whose stride is not a multiple of 16 bytes are read whole in every mode."""
    cat = synth.catalog(40_000, 3, ("zipf",) * 3, [74, 1])
    widths = [7, 128, 512]
    runs = [gh.Run(cat, widths, read_mode=m) for m in ("dense", "gather")]
    for t in range(3):
        dev = _pack(runs[0], gh.rowkeyed_logits(74, t, widths, 2.0, False), False, ld=257)
        states = []
        for r in runs:
            r.beams.step(dev)
            states.append(r.state())
        _bitwise(runs[0], states[0], states[1], t, "gather")


def _two_branch_catalog():
    """Root children {3, 200}; every second code under each."""
    a = np.repeat(np.asarray([3, 200], dtype=np.uint8), 256)
    b = np.tile(np.arange(256, dtype=np.uint8), 2)
    return np.stack([a, b], axis=1)


@pytest.mark.parametrize("mode,code,expect_error", [
    ("gather", 3, True),      # a child's logit is always checked
    ("dense", 100, True),     # whole rows are checked
    ("gather", 100, False),   # the piece of codes 100..103 holds no child and is not read
])
def test_gather_validate(mode, code, expect_error):
    from trie_constrained_beam_amd import TcbError
    run = gh.Run(_two_branch_catalog(), [16], read_mode=mode)
    run.beams.set_validate(True)
    x = torch.zeros((16, 256), device="cuda")
    x[0, code] = float("nan")
    run.beams.step(x)
    if expect_error:
        with pytest.raises(TcbError, match="NONFINITE"):
            run.beams.check()
    else:
        run.beams.check()
