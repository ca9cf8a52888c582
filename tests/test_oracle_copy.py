"""Pins of the copy-draft reference (oracle/copy_draft.py).

Worked examples follow the definition on the pages (model card, section Use:
copy drafts from the context are tried first; page 2, the frozen-corpus
article: longest suffix 8 down to 3, most recent occurrence, spans of up to K
tokens that never cross a -1 separator; the 24-proposal, 50 %, 256-token pause
guard). A second, vectorised formulation (the longest match length at every
position, then the latest position with it) must agree on random inputs.
"""
import numpy as np
import pytest

from oracle.copy_draft import PauseGuard, copy_draft


def test_worked_examples():
    # the 4-token suffix 5 6 7 8 occurred at the start: propose what followed
    t = [5, 6, 7, 8, 9, 1, 2, 3, 5, 6, 7, 8]
    assert copy_draft(t, len(t), None, 4) == ([9, 1, 2, 3], 4, "context")
    # K caps the span; the context end caps it too
    assert copy_draft(t, len(t), None, 2) == ([9, 1], 4, "context")
    t2 = [1, 2, 3, 4, 1, 2, 3]
    assert copy_draft(t2, len(t2), None, 8) == ([4, 1, 2, 3], 3, "context")
    # the most recent of two occurrences wins
    t3 = [7, 8, 9, 1, 7, 8, 9, 2, 7, 8, 9]
    assert copy_draft(t3, len(t3), None, 3) == ([2, 7, 8], 3, "context")
    # a longer suffix beats a more recent shorter one
    t4 = [1, 2, 3, 4, 5, 0, 2, 3, 4, 6, 1, 2, 3, 4]
    assert copy_draft(t4, len(t4), None, 2) == ([5, 0], 4, "context")
    # the suffix itself is no occurrence; fewer than 3 tokens never propose
    assert copy_draft([1, 2, 3, 4], 4, None, 4) == ([], 0, None)
    assert copy_draft([3, 3], 2, None, 4) == ([], 0, None)
    assert copy_draft([], 0, [1, 2, 3], 4) == ([], 0, None)
    # a run of one token matches itself shifted by one
    assert copy_draft([4, 4, 4, 4, 4], 5, None, 3) == ([4], 4, "context")


def test_corpus_examples():
    c = [9, 1, 2, 3, 4, 7, 7, -1, 2, 3, 4, 8]
    # context misses; the corpus holds the 4-token suffix; the span stops at -1
    assert copy_draft([1, 2, 3, 4], 4, c, 3) == ([7, 7], 4, "corpus")
    # a match followed by a separator or the corpus end is no proposal
    assert copy_draft([6, 2, 3, 4, 8], 5, [0, 2, 3, 4, 8, -1], 3) == ([], 0, None)
    assert copy_draft([6, 2, 3, 4, 8], 5, [0, 2, 3, 4, 8], 3) == ([], 0, None)
    # matches never span a separator
    assert copy_draft([5, 1, 2, 3], 4, [1, -1, 2, 3, 9], 3) == ([], 0, None)
    assert copy_draft([5, 1, 2, 3], 4, [1, 2, 3, 9], 3) == ([9], 3, "corpus")
    # at equal length the context is tried first; a longer corpus match wins
    assert copy_draft([1, 2, 3, 5, 1, 2, 3], 7, [1, 2, 3, 6], 3) == ([5, 1, 2], 3, "context")
    assert copy_draft([1, 2, 3, 8, 5, 1, 2, 3], 8, [0, 5, 1, 2, 3, 6], 3) == ([6], 4, "corpus")


def _vectorised(tokens, length, corpus, K):
    """Longest match m(p) <= 8 ending before every candidate position p,
    then the latest p with the largest m (context first at equal m)."""
    t = np.asarray(tokens[:length], dtype=np.int64)
    suf = t[max(0, length - 8):]

    def best(seq, ok):
        n = len(seq)
        m = np.zeros(n + 1, dtype=np.int64)
        alive = np.ones(n + 1, dtype=bool)
        for i in range(len(suf)):
            pos = np.arange(n + 1) - 1 - i
            hit = np.zeros(n + 1, dtype=bool)
            inb = pos >= 0
            hit[inb] = seq[pos[inb]] == suf[len(suf) - 1 - i]
            alive &= hit
            m += alive
        m[~ok] = 0
        top = m.max(initial=0)
        if top < 3:
            return 0, -1
        return int(top), int(np.nonzero(m == top)[0].max())

    okc = np.zeros(len(t) + 1, dtype=bool)
    okc[1:len(t)] = True                          # a continuation exists
    mc, pc = best(t, okc)
    c = np.asarray([] if corpus is None else corpus, dtype=np.int64)
    oko = np.zeros(len(c) + 1, dtype=bool)
    if len(c):
        oko[1:len(c)] = c[1:] != -1
    mo, po = best(c, oko)
    if max(mc, mo) < 3:
        return [], 0, None
    if mc >= mo:
        return [int(x) for x in t[pc:min(pc + K, length)]], mc, "context"
    span = []
    for x in c[po:po + K]:
        if x == -1:
            break
        span.append(int(x))
    return span, mo, "corpus"


@pytest.mark.parametrize("seed", range(40))
def test_agrees_with_vectorised_formulation(seed):
    rng = np.random.default_rng(seed)
    alpha = int(rng.integers(2, 6))
    L = int(rng.integers(0, 60))
    t = rng.integers(0, alpha, size=L).tolist()
    corpus = None
    if seed % 3:
        corpus = rng.integers(0, alpha, size=int(rng.integers(0, 80))).tolist()
        for i in rng.integers(0, max(len(corpus), 1), size=3):
            if len(corpus):
                corpus[int(i)] = -1
    K = int(rng.integers(1, 10))
    assert copy_draft(t, L, corpus, K) == _vectorised(t, L, corpus, K)


def test_pause_guard():
    g = PauseGuard()
    for _ in range(23):
        g.record(4, 1)                 # 25 % so far, but the window is not full
        assert g.armed()
    g.record(4, 1)                     # 24 proposals at 25 % < 50 %: pause
    assert not g.armed()
    g.advance(255)
    assert not g.armed()
    g.advance(1)                       # 256 tokens later: re-armed, window empty
    assert g.armed()
    for _ in range(24):
        g.record(4, 2)                 # exactly 50 % keeps the source armed
    assert g.armed()
    g.record(4, 0)                     # the window slides: 23 x 2 + 0 = 46 of 96 < 50 %
    assert not g.armed()
