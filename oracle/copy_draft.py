"""Copy (suffix-match) drafts, plain CPU reference.

TEST INFRASTRUCTURE ONLY: imported by the tests; never by the library.

Authority: the model card "Kolibri-1 block drafter", section Use: copy drafts
from the context are tried before the learned block. The article on
Colibri's frozen-corpus drafts (page 2, "它解决什么问题" and "第二步"): each
step proposes the continuation that follows the longest suffix of the current
context, suffix length 8 down to 3, taking the most recent occurrence; a hit
proposes a whole span of up to K tokens (default 8, at most 48); the corpus is
token ids with -1 separating spans and a proposal never crosses a separator;
the pause guard ("语料近邻的风险") stops the source for 256 tokens when fewer
than 50 % of the last 24 proposals were accepted, then re-arms it.

Readings where the pages are silent:
* the sources are the stream's own context and an optional frozen corpus; at
  each suffix length (longest first) the context is tried before the corpus;
* an occurrence counts only if at least one token follows it: in the context a
  match ending at the last token (the suffix itself) is not a proposal, in the
  corpus the following token must not be a separator;
* the proposal is the tokens after the occurrence, up to K, stopping at the
  end of the context (context source) or at a separator or the corpus end;
* the guard counts proposed and accepted tokens per proposal; a proposal with
  no accepted token counts as rejected.
"""
from __future__ import annotations

import numpy as np

S_MAX, S_MIN = 8, 3


def _last_occurrence(seq, suffix, limit, follows):
    """Largest p with s <= p < limit, seq[p - s:p] == suffix and follows(p);
    -1 if none."""
    s = len(suffix)
    for p in range(limit - 1, s - 1, -1):
        if all(seq[p - s + i] == suffix[i] for i in range(s)) and follows(p):
            return p
    return -1


def copy_draft(tokens, length, corpus, K):
    """Returns (proposal list, suffix length, source) for one stream; source is
    "context", "corpus" or None (no proposal, suffix length 0)."""
    t = [int(x) for x in tokens[:length]]
    c = [] if corpus is None else [int(x) for x in corpus]
    for s in range(S_MAX, S_MIN - 1, -1):
        if length < s:
            continue
        suffix = t[length - s:]
        # context: the occurrence ends before the last token, so a
        # continuation exists
        p = _last_occurrence(t, suffix, length, lambda p: True)
        if p >= 0:
            return t[p:min(p + K, length)], s, "context"
        # corpus: the next token exists and is not a separator
        q = _last_occurrence(c, suffix, len(c), lambda q: c[q] != -1)
        if q >= 0:
            out = []
            for tok in c[q:q + K]:
                if tok == -1:
                    break
                out.append(tok)
            return out, s, "corpus"
    return [], 0, None


class PauseGuard:
    """The acceptance pause guard: over the last `window` proposals, if the
    accepted share of proposed tokens is below `min_acc`, the source pauses for
    `pause` tokens of decoding, then re-arms with an empty window."""

    def __init__(self, window=24, min_acc=0.5, pause=256):
        self.window, self.min_acc, self.pause = window, min_acc, pause
        self.hist = []          # (proposed, accepted) of recent proposals
        self.paused_left = 0

    def armed(self):
        return self.paused_left == 0

    def record(self, proposed, accepted):
        """A proposal of `proposed` tokens of which `accepted` were kept."""
        self.hist.append((proposed, accepted))
        if len(self.hist) > self.window:
            self.hist.pop(0)
        if len(self.hist) == self.window:
            p = sum(h[0] for h in self.hist)
            a = sum(h[1] for h in self.hist)
            if p > 0 and a < self.min_acc * p:
                self.paused_left = self.pause
                self.hist = []

    def advance(self, tokens):
        """`tokens` tokens were decoded (with or without proposals)."""
        self.paused_left = max(0, self.paused_left - tokens)
