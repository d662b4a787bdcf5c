"""The scoring entry point that allocates nothing (tcb_score_catalog_static, the library's
static scratch) against tcb_score_catalog with a caller workspace: bitwise equal results
on two calls in a row, the second smaller (fewer users, smaller k, no SID-level term), so
the second reads scratch the first left behind; and a call that needs more scratch than
the static array holds is refused before anything is launched."""
import numpy as np
import pytest
import torch

from trie_constrained_beam_amd import Trie, TcbError, score_catalog, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    print(f"\n[gpu] {request.node.name}", flush=True)


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _same(a, b, ctx):
    for key in ("leaf", "item", "score", "lse"):
        if a[key] is None:
            assert b[key] is None, (ctx, key)
            continue
        x, y = a[key].cpu().numpy(), b[key].cpu().numpy()
        assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                              y.view(np.uint32) if y.dtype == np.float32 else y), (ctx, key)


def test_static_scratch_matches_workspace():
    cat = synth.catalog(300_000, 4, ("uniform",) + ("zipf",) * 3, [81, 1])
    trie = Trie(cat, device="cuda").upload_codes("cuda")
    cases = [(32, 512, 64, "logits"), (5, 50, 0, "logprob")]     # the second call is smaller
    for users, k, dim, kind in cases:
        table = torch.from_numpy(synth.score_logits(81 + users, users, trie.L, 2.0)).cuda()
        if kind == "logprob":
            table = torch.log_softmax(table, dim=-1).contiguous()
        uv = em = None
        if dim:
            uv = _bf16(synth.user_vectors(81, users, dim))
            em = _bf16(synth.sid_embeddings(81, trie.n_distinct, dim))
        ref = score_catalog(trie, table, k, kind, uv, em, 0.7)
        dev = table.device
        out = {"leaf": torch.full((users, k), -5, dtype=torch.int32, device=dev),
               "item": torch.full((users, k), -5, dtype=torch.int32, device=dev),
               "score": torch.full((users, k), 9.0, dtype=torch.float32, device=dev),
               "lse": torch.full((users,), 9.0, dtype=torch.float32, device=dev)}
        got = score_catalog(trie, table, k, kind, uv, em, 0.7, workspace="static", out=out)
        torch.cuda.synchronize()
        _same(ref, got, (users, k, dim))


def test_static_scratch_refuses_oversize_calls():
    cat = synth.catalog(300_000, 4, ("zipf",) * 4, [82, 1])
    trie = Trie(cat, device="cuda").upload_codes("cuda")
    users = 4096                                       # ~300 MB of scratch: more than 64 MiB
    table = torch.zeros((users, trie.L, 256), dtype=torch.float32, device="cuda")
    out = {"leaf": torch.empty((users, 8), dtype=torch.int32, device="cuda"),
           "item": torch.empty((users, 8), dtype=torch.int32, device="cuda"),
           "score": torch.empty((users, 8), dtype=torch.float32, device="cuda"), "lse": None}
    with pytest.raises(TcbError, match="WORKSPACE"):
        score_catalog(trie, table, 8, "logits", workspace="static", out=out)
