"""Single-pass scoring of every valid SID on the GPU against the oracle: per-user top-k
(windowed near-ties), scores, catalog items and the log-normaliser over valid SIDs."""
import ctypes as C

import numpy as np
import pytest
import torch

import gpu_harness as gh
import oracle
from trie_constrained_beam_amd import Trie, TcbError, score_catalog, synth
from trie_constrained_beam_amd import _lib as L

pytestmark = pytest.mark.gpu


def _run(cat, V, table, kind, k, uvec=None, emb=None, w=1.0, users=None, want_lse=True, trie=None):
    """GPU scoring of every user, oracle comparison for ``users`` (default: all)."""
    trie = trie or Trie(cat, V=V, device="cuda")
    otrie = oracle.OracleTrie(cat.astype(np.int64), V=V)
    dt = torch.from_numpy(table).cuda()
    du = torch.from_numpy(uvec.view(np.int16)).cuda().view(torch.bfloat16) if uvec is not None else None
    de = torch.from_numpy(emb.view(np.int16)).cuda().view(torch.bfloat16) if emb is not None else None
    out = score_catalog(trie, dt, k, kind, du, de, w, want_lse=want_lse)
    torch.cuda.synchronize()
    res = {key: (v.cpu().numpy() if v is not None else None) for key, v in out.items()}
    u64 = oracle.widen_logits(uvec, "bf16") if uvec is not None else None
    e64 = oracle.widen_logits(emb, "bf16") if emb is not None else None
    okind = oracle.TABLE_LOGITS if kind == "logits" else oracle.TABLE_LOGPROB
    for u in (range(table.shape[0]) if users is None else users):
        ref = oracle.score_catalog(otrie, table[u].astype(np.float64), k, okind,
                                   u64[u] if u64 is not None else None, e64, w)
        gh.compare_topk(ref["all_scores"], res["leaf"][u], res["score"][u], k, ctx=f"user {u}")
        kk = min(k, otrie.n_distinct)
        assert np.array_equal(res["item"][u][:kk], otrie.leaf_item[res["leaf"][u][:kk]])
        assert (res["item"][u][kk:] == -1).all()
        if want_lse:
            assert abs(float(res["lse"][u]) - ref["lse"]) <= 1e-4, (u, res["lse"][u], ref["lse"])
    return res


def test_score_token_only_logprob():
    cat = synth.catalog(20_000, 3, ("uniform",) * 3, [80, 1])
    _run(cat, 256, synth.score_logprobs(80, 5, 3), "logprob", 50)


def test_score_logits_with_sid_term_ragged_users():
    """37 users: a full group of 32 and a ragged one."""
    cat = synth.catalog(60_000, 4, ("zipf",) * 4, [81, 1])
    n = len(np.unique(synth.pack_sids(cat)))
    _run(cat, 256, synth.score_logits(81, 37, 4), "logits", 100,
         synth.user_vectors(81, 37, 64), synth.sid_embeddings(81, n, 64), 0.7)


@pytest.mark.parametrize("D", [32, 128, 256])
def test_score_dims(D):
    cat = synth.catalog(30_000, 4, ("uniform",) + ("zipf",) * 3, [82, D])
    n = len(np.unique(synth.pack_sids(cat)))
    _run(cat, 256, synth.score_logits(82, 3, 4), "logits", 20,
         synth.user_vectors(82, 3, D), synth.sid_embeddings(82, n, D), 1.3)


@pytest.mark.parametrize("Ld,n_cat", [(5, 30_000), (8, 10_000)])
def test_score_deep_sids(Ld, n_cat):
    """L > 4: 8-byte codes and groups of 16 users (20 users: two groups)."""
    cat = synth.catalog(n_cat, Ld, ("uniform",) * Ld, [83, Ld])
    n = len(np.unique(synth.pack_sids(cat)))
    _run(cat, 256, synth.score_logits(83, 20, Ld), "logits", 10,
         synth.user_vectors(83, 20, 32), synth.sid_embeddings(83, n, 32), 0.5)


def test_score_k_above_catalog_and_single_sid():
    cat = synth.catalog(300, 2, ("uniform",) * 2, [84, 1])
    _run(cat, 256, synth.score_logits(84, 4, 2), "logits", 512)
    one = np.asarray([[7, 9, 11]], dtype=np.uint8)
    _run(one, 256, synth.score_logits(85, 2, 3), "logits", 3)


def test_score_k_one_and_small_codebook():
    cat = synth.catalog(5_000, 3, ("uniform",) * 3, [86, 1], V=50)
    n = len(np.unique(synth.pack_sids(cat)))
    tab = synth.score_logits(86, 6, 3, V=50)
    _run(cat, 50, tab, "logits", 1, synth.user_vectors(86, 6, 64), synth.sid_embeddings(86, n, 64), 1.0)
    _run(cat, 50, tab, "logits", 33)


def test_score_exact_ties():
    """Integer log-probabilities make every fp32 sum exact, with many equal scores: the
    whole top-k (ties by ascending SID) must equal the oracle's exactly."""
    cat = synth.catalog(50_000, 4, ("zipf",) * 4, [87, 1])
    rng = np.random.default_rng([87, 2])
    tab = -rng.integers(0, 4, (6, 4, 256)).astype(np.float32)
    tab[5] = -1.0                                        # one user: every SID tied
    trie = Trie(cat, device="cuda")
    res = _run(cat, 256, tab, "logprob", 300, trie=trie)
    otrie = oracle.OracleTrie(cat.astype(np.int64))
    for u in range(6):
        ref = oracle.score_catalog(otrie, tab[u].astype(np.float64), 300, oracle.TABLE_LOGPROB)
        assert np.array_equal(res["leaf"][u], ref["leaf"]), u
        assert np.array_equal(res["score"][u], ref["score"].astype(np.float32)), u
    assert np.array_equal(res["leaf"][5], np.arange(300))


def test_score_lse_off_and_determinism():
    cat = synth.catalog(40_000, 4, ("zipf",) * 4, [88, 1])
    n = len(np.unique(synth.pack_sids(cat)))
    trie = Trie(cat, device="cuda")
    tab = torch.from_numpy(synth.score_logits(88, 33, 4)).cuda()
    uv = torch.from_numpy(synth.user_vectors(88, 33, 64).view(np.int16)).cuda().view(torch.bfloat16)
    em = torch.from_numpy(synth.sid_embeddings(88, n, 64).view(np.int16)).cuda().view(torch.bfloat16)
    outs = [score_catalog(trie, tab, 200, "logits", uv, em, 0.9, want_lse=f) for f in (True, True, False)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o["leaf"], outs[0]["leaf"])
        assert torch.equal(o["score"].view(torch.int32), outs[0]["score"].view(torch.int32))
        assert torch.equal(o["item"], outs[0]["item"])
    assert torch.equal(outs[1]["lse"].view(torch.int32), outs[0]["lse"].view(torch.int32))


def test_score_fullsize_sampled_users():
    """The 4M-SID Zipf catalog, 32 users, 64-dim SID term, top 512 (the measured
    configuration); three users checked against the oracle over every SID."""
    wl = synth.SCORE_WORKLOADS["score_u32_k512_l4_4m_zipf_d64"]
    cat = wl.catalog()
    trie = Trie(cat, device="cuda")
    n = trie.n_distinct
    _run(cat, 256, synth.score_logits(wl.seed, wl.users, 4, wl.sigma), "logits", wl.k,
         synth.user_vectors(wl.seed, wl.users, wl.dim), synth.sid_embeddings(wl.seed, n, wl.dim), 1.0,
         users=[0, 17, 31], trie=trie)


def test_score_superblock_path():
    """More than 16384 blocks of 256 SIDs: the pick goes through superblocks. 16384 * 256 + 1
    SIDs (every 4-byte code below that count), so the last superblock holds one block of
    one SID; a SID-level term and a ragged user group."""
    n = 16384 * 256 + 1
    i = np.arange(n, dtype=np.uint32)
    cat = np.stack([(i >> 24) & 255, (i >> 16) & 255, (i >> 8) & 255, i & 255], axis=1).astype(np.uint8)
    trie = Trie(cat, device="cuda")
    assert trie.n_distinct == n
    _run(cat, 256, synth.score_logits(90, 3, 4), "logits", 300,
         synth.user_vectors(90, 3, 32), synth.sid_embeddings(90, n, 32), 0.8, trie=trie)


def test_score_argument_errors():
    cat = synth.catalog(2_000, 3, ("uniform",) * 3, [89, 1])
    trie = Trie(cat, device="cuda")
    tab = torch.zeros((2, 3, 256), device="cuda")
    with pytest.raises(TcbError, match="STATE"):          # codes not uploaded
        nb = 1 << 20
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        out = torch.empty((2, 4), dtype=torch.int32, device="cuda")
        sc = torch.empty((2, 4), device="cuda")
        L.check(L.lib().tcb_score_catalog(trie.handle, 2, C.c_void_p(tab.data_ptr()), 0, None, None, 0,
                                          1.0, 4, C.c_void_p(out.data_ptr()), None, C.c_void_p(sc.data_ptr()),
                                          None, C.c_void_p(ws.data_ptr()), nb, None))
    trie.upload_codes()
    uv = torch.zeros((2, 48), dtype=torch.bfloat16, device="cuda")
    em = torch.zeros((trie.n_distinct, 48), dtype=torch.bfloat16, device="cuda")
    for kw, msg in [(dict(k=0), "TCB_E_ARG"), (dict(k=513), "k must"),
                    (dict(k=4, user_vec=uv, sid_emb=em), "dim must")]:
        with pytest.raises(TcbError, match=msg):
            score_catalog(trie, tab, **kw)
    with pytest.raises(ValueError):
        score_catalog(trie, tab, 4, user_vec=uv[:, :32].contiguous())
    with pytest.raises(TcbError, match="WORKSPACE"):
        score_catalog(trie, tab, 4, workspace=torch.empty(1 << 20, dtype=torch.uint8, device="cuda")[1:])
