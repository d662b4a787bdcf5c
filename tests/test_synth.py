"""Seeded input generators: determinism, distinctness, and known values. CPU only."""
import numpy as np
import torch

from trie_constrained_beam_amd import synth


def test_splitmix64_known_value():
    # SplitMix64 seeded with 0: first output 0xE220A8397B1DCDAF (published reference stream)
    assert int(synth.splitmix64(np.uint64(0))) == 0xE220A8397B1DCDAF
    assert int(synth.splitmix64(np.uint64(0x9E3779B97F4A7C15))) == 0x6E789E6AA1B965F4


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 3, 10000), rng.normal(0, 1e-3, 1000),
                        [0.0, -0.0, 1.0, 3.0000001, 1.00390625, 1.01171875]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(x), ref)
    back = synth.bf16_bits_to_f32(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_catalog_distinct_first_occurrence_and_deterministic():
    a = synth.catalog(5000, 3, ("uniform", "zipf", "zipf"), [9, 1])
    b = synth.catalog(5000, 3, ("uniform", "zipf", "zipf"), [9, 1])
    assert a.shape == (5000, 3) and a.dtype == np.uint8
    assert np.array_equal(a, b)
    keys = synth.pack_sids(a)
    assert np.unique(keys).size == 5000
    # Zipf levels: code 0 is the most frequent
    counts = np.bincount(a[:, 1], minlength=256)
    assert counts.argmax() == 0


def test_logits_generators_deterministic():
    x1 = synth.logits_rowkeyed(3, 1, 7, 16, 3.0)
    x2 = synth.logits_rowkeyed(3, 1, 7, 16, 3.0)
    assert x1.dtype == np.float32 and x1.shape == (16, 256) and np.array_equal(x1, x2)
    assert abs(float(x1.std()) - 3.0) < 0.2
    b = synth.logits_rowkeyed(3, 1, 7, 16, 3.0, bf16=True)
    assert b.dtype == np.uint16 and np.array_equal(b, synth.f32_to_bf16_bits(x1))
    p = synth.logits_prefixkeyed(11, 2, [5, 6, 5], 2.0)
    assert p.shape == (3, 256) and np.array_equal(p[0], p[2]) and not np.array_equal(p[0], p[1])
    assert np.array_equal(p[1:2], synth.logits_prefixkeyed(11, 2, [6], 2.0))


def test_workload_table():
    w = synth.WORKLOADS
    assert w["b512x32_l4_4m_zipf_bf16"].widths == (512,) * 32
    mixed = w["mixed256_l5_8m_f32"]
    assert len(mixed.widths) == 256 and set(mixed.widths) <= {50, 128, 256, 512}


def test_catalog_refuses_more_sids_than_exist():
    import pytest
    with pytest.raises(ValueError):
        synth.catalog(70_000, 2, ("uniform", "uniform"), [1, 1])
