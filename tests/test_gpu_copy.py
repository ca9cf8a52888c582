"""Copy (suffix-match) drafts on the GPU against the CPU reference
(oracle/copy_draft.py), bit for bit: proposed ids, counts, suffix lengths and
sources. Inputs are seeded and synthetic: token histories and corpora over
small alphabets (so suffixes recur), separators in the corpus, ragged and
out-of-range lengths, K from 1 to the limit."""
import time

import numpy as np
import pytest
import torch

from block_draft_model_amd import kdraft
from gpu_common import log, require_gpu
from oracle.copy_draft import copy_draft
from test_oracle_copy import _vectorised

pytestmark = pytest.mark.gpu

SRC = {None: 0, "context": 1, "corpus": 2}


@pytest.fixture(scope="module")
def dr():
    require_gpu()
    d = kdraft.Drafter(max_streams=256)
    yield d
    d.close()


def run(dr, tokens, lens, corpus, K):
    B, stride = tokens.shape
    t = torch.from_numpy(np.ascontiguousarray(tokens, dtype=np.int32)).cuda()
    ln = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    c = None if corpus is None else torch.from_numpy(np.asarray(corpus, dtype=np.int32)).cuda()
    ids = torch.full((B, K), -7, dtype=torch.int32, device="cuda")
    info = torch.full((B, 3), -7, dtype=torch.int32, device="cuda")
    dr.copy_draft(B, t, stride, ln, c, 0 if corpus is None else len(corpus), K, ids, info)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), info.cpu().numpy()


def expect(tokens, lens, corpus, K, ref=copy_draft):
    B, stride = tokens.shape
    ids = np.full((B, K), -1, dtype=np.int32)
    info = np.zeros((B, 3), dtype=np.int32)
    for b in range(B):
        L = int(min(max(int(lens[b]), 0), stride))
        span, s, src = ref(tokens[b].tolist(), L, corpus, K)
        ids[b, :len(span)] = span
        info[b] = (len(span), s, SRC[src])
    return ids, info


@pytest.mark.parametrize("seed", range(6))
def test_copy_drafts_match_reference(dr, seed):
    rng = np.random.default_rng(100 + seed)
    B, stride = 24, 160
    alpha = 2 + seed % 4
    tokens = rng.integers(0, alpha, size=(B, stride)).astype(np.int32)
    lens = rng.integers(0, stride + 1, size=B)
    lens[:6] = [0, 1, 2, 3, stride, stride + 40]      # edges; the last is clamped to stride
    lens[6] = -5                                        # clamped to 0
    corpus = None
    if seed % 3:
        corpus = rng.integers(0, alpha + 1, size=400).astype(np.int32)
        corpus[rng.integers(0, 400, size=12)] = -1
    for K in (1, 7, kdraft.KD_MAX_COPY):
        got_ids, got_info = run(dr, tokens, lens, corpus, K)
        want_ids, want_info = expect(tokens, lens, corpus, K)
        assert np.array_equal(got_info, want_info), (seed, K)
        assert np.array_equal(got_ids, want_ids), (seed, K)
    log(f"seed {seed}: sources {np.bincount(got_info[:, 2], minlength=3).tolist()}")


def test_copy_drafts_large_corpus(dr):
    # 64 histories of 2048 tokens over a 1,000-token alphabet and a 1M-id
    # corpus with each stream's last 5..8 tokens planted at random places
    rng = np.random.default_rng(7)
    B, stride, N = 64, 2048, 1 << 20
    tokens = rng.integers(0, 1000, size=(B, stride)).astype(np.int32)
    lens = rng.integers(1500, stride + 1, size=B)
    corpus = rng.integers(0, 1000, size=N).astype(np.int32)
    corpus[rng.integers(0, N, size=2000)] = -1
    for b in range(B):
        s = int(rng.integers(5, 9))
        at = int(rng.integers(s, N - 20))
        corpus[at - s:at] = tokens[b, lens[b] - s:lens[b]]
        corpus[at] = max(int(corpus[at]), 0)
    K = 8
    got_ids, got_info = run(dr, tokens, lens, corpus, K)
    want_ids, want_info = expect(tokens, lens, corpus.tolist(), K, ref=_vectorised)
    assert np.array_equal(got_info, want_info)
    assert np.array_equal(got_ids, want_ids)
    # time it (the histories and the corpus are resident)
    t = torch.from_numpy(tokens).cuda()
    ln = torch.from_numpy(lens.astype(np.int32)).cuda()
    c = torch.from_numpy(corpus).cuda()
    ids = torch.empty((B, K), dtype=torch.int32, device="cuda")
    info = torch.empty((B, 3), dtype=torch.int32, device="cuda")
    for _ in range(3):
        dr.copy_draft(B, t, stride, ln, c, N, K, ids, info)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(20):
        dr.copy_draft(B, t, stride, ln, c, N, K, ids, info)
    torch.cuda.synchronize()
    log(f"copy drafts: {B} streams x {stride}-token histories + {N}-id corpus: "
        f"{(time.perf_counter() - t0) / 20 * 1e6:.1f} us per call; "
        f"sources {np.bincount(got_info[:, 2], minlength=3).tolist()}")
