"""kd_copy_draft_noalloc (the copy-draft call that allocates nothing, for
callers that cannot allocate device memory) against kd_copy_draft, bit for
bit: two calls in a row on one stream, the second with fewer streams and a
shorter corpus, so that it reuses the fixed key array the first one filled.
Inputs are seeded and synthetic (small alphabets so suffixes recur, corpus
separators, ragged lengths)."""
import numpy as np
import pytest
import torch

from block_draft_model_amd import kdraft
from gpu_common import log, require_gpu

pytestmark = pytest.mark.gpu


def _case(seed, B, stride, corpus_len, alpha):
    rng = np.random.default_rng(seed)
    tokens = rng.integers(0, alpha, size=(B, stride)).astype(np.int32)
    lens = rng.integers(0, stride + 1, size=B).astype(np.int32)
    lens[:3] = [0, 3, stride]
    corpus = rng.integers(0, alpha + 1, size=corpus_len).astype(np.int32)
    corpus[rng.integers(0, corpus_len, size=corpus_len // 40)] = -1
    dev = lambda a: torch.from_numpy(a).cuda()
    return dev(tokens), stride, dev(lens), dev(corpus), corpus_len


def _outputs(B, K):
    return (torch.full((B, K), -7, dtype=torch.int32, device="cuda"),
            torch.full((B, 3), -7, dtype=torch.int32, device="cuda"))


def test_noalloc_copy_drafts_equal_the_context_call():
    require_gpu()
    dr = kdraft.Drafter(max_streams=256)
    try:
        cases = [(_case(501, 200, 512, 6000, 3), 200, 11), (_case(502, 24, 160, 700, 2), 24, 5)]
        got = []
        for (t, stride, ln, c, n), B, K in cases:   # both calls enqueued before any sync
            ids, info = _outputs(B, K)
            assert kdraft.copy_draft_noalloc(B, t, stride, ln, c, n, K, ids, info) == kdraft.KD_OK
            got.append((ids, info))
        for ((t, stride, ln, c, n), B, K), (ids, info) in zip(cases, got):
            want_ids, want_info = _outputs(B, K)
            dr.copy_draft(B, t, stride, ln, c, n, K, want_ids, want_info)
            torch.cuda.synchronize()
            src = np.bincount(info[:, 2].cpu().numpy(), minlength=3).tolist()
            log(f"B={B} K={K}: sources {src}")
            assert torch.equal(info, want_info)
            assert torch.equal(ids, want_ids)
            assert src[1] > 0 and src[2] > 0   # both sources win somewhere
    finally:
        dr.close()


def test_noalloc_copy_draft_rejects_more_streams_than_its_array():
    require_gpu()
    B = kdraft.KD_COPY_NOALLOC_MAX_STREAMS + 1
    t = torch.zeros((B, 8), dtype=torch.int32, device="cuda")
    ln = torch.zeros(B, dtype=torch.int32, device="cuda")
    ids, info = _outputs(B, 4)
    assert kdraft.copy_draft_noalloc(B, t, 8, ln, None, 0, 4, ids, info) == kdraft.KD_ERR_ARG
    assert kdraft.copy_draft_noalloc(0, t, 8, ln, None, 0, 4, ids, info) == kdraft.KD_ERR_ARG
    torch.cuda.synchronize()
    assert int(info.min()) == -7   # nothing was launched
