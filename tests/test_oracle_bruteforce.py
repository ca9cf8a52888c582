"""Brute force: the whole round, and ingest, written as explicit Python loops on
a tiny model, against the oracle.

Weights are decoded through lookup tables taken from torch's float8_e4m3fn and
bfloat16 casts and from the OCP e2m1 value list, not through the oracle's
decoders; every product is an explicit loop with W[out][in] indexing. The
steps follow the model card ("Kolibri-1 block drafter", Architecture) in the
same readings the oracle states.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

D = synth.TINY
E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().tolist()
E2M1 = [float(v) for v in np.loadtxt(os.path.join(os.path.dirname(__file__), "golden",
                                                  "e2m1_values.txt"))[:, 1]]
E2M1 = E2M1 + [-v for v in E2M1]


def bf16(bits):
    return torch.tensor(int(bits) - 65536 if bits >= 32768 else int(bits),
                        dtype=torch.int16).view(torch.bfloat16).item()


def fp8_matrix(m, name):
    q, s = m[name + ".q"], m[name + ".s"]
    rows, cols = q.shape
    return [[E4M3[int(q[o, i])] * float(s[o, i // 64]) for i in range(cols)] for o in range(rows)]


def mv(W, x):
    return [sum(w * xi for w, xi in zip(row, x)) for row in W]


def rms(x, g):
    r = math.sqrt(sum(v * v for v in x) / len(x) + D.rms_eps)
    return [gi * v / r for gi, v in zip(g, x)]


def silu(v):
    return v / (1.0 + math.exp(-v))


def rope(vec, p):
    half = len(vec) // 2
    out = list(vec)
    for i in range(half):
        ang = p * D.rope_theta ** (-i / half)
        c, s = math.cos(ang), math.sin(ang)
        out[i] = vec[i] * c - vec[i + half] * s
        out[i + half] = vec[i] * s + vec[i + half] * c
    return out


class Brute:
    def __init__(self, m):
        # fp32 vectors become Python floats (exact), so no float32 arithmetic
        # leaks in through numpy scalars
        self.m = {k: (v.astype(np.float64).tolist()
                      if isinstance(v, np.ndarray) and v.dtype == np.float32 and v.ndim == 1 else v)
                  for k, v in m.items()}
        m = self.m
        self.W = {}
        for key in m:
            if key.endswith(".q"):
                self.W[key[:-2]] = fp8_matrix(m, key[:-2])
        q4, s4, g = m["head.q4"], m["head.s4"], float(np.float32(m["head.g"]))
        self.head = []
        for o in range(q4.shape[0]):
            row = []
            for i in range(D.hidden):
                byte = int(q4[o, i // 2])
                code = byte & 0xF if i % 2 == 0 else byte >> 4
                row.append(E2M1[code] * E4M3[int(s4[o, i // 16])] * g)
            self.head.append(row)

    def embed(self, tok):
        return [bf16(b) for b in self.m["table"][int(tok)]]

    def context_kv(self, layer, kcache, vcache, length):
        n = min(length, D.window)
        ks, vs = [], []
        for p in range(length - n, length):
            slot = p % D.capacity
            ks.append([[bf16(b) for b in kcache[h, slot]] for h in range(D.heads)])
            vs.append([[bf16(b) for b in vcache[h, slot]] for h in range(D.heads)])
        return ks, vs

    def round_one(self, taps, anchor, pred, length, kcaches, vcaches):
        m, W, H = self.m, self.W, D.hidden
        t = [bf16(b) for b in taps.reshape(-1)]
        f = mv(W["fuse"], t)
        x = [mv(W["fc"], f + self.embed(anchor))]
        for j in range(1, 4):
            e = self.embed(pred[j - 1])
            u = [a + b for a, b in zip(mv(W["pred_a"], f), mv(W["pred_b"], e))]
            add = mv(W["pred_u"], [silu(v) for v in u])
            x.append([mk + fi + ad for mk, fi, ad in zip(m["mask"], f, add)])
        for l in range(D.layers):
            p = f"layers.{l}."
            if l >= 1:
                sp = f"spine.{l}."
                prev = [list(r) for r in x]
                for j in range(1, 4):
                    a = rms(prev[j - 1], m[sp + "norm"])
                    add = mv(W[sp + "u"], [silu(v) for v in mv(W[sp + "a"], a)])
                    x[j] = [xv + av for xv, av in zip(prev[j], add)]
            q, k, v = [], [], []
            for j in range(4):
                a = rms(x[j], m[p + "attn_norm"])
                qq, kk, vv = mv(W[p + "wq"], a), mv(W[p + "wk"], a), mv(W[p + "wv"], a)
                dh = D.head_dim
                q.append([rope(qq[h * dh:(h + 1) * dh], length + j) for h in range(D.heads)])
                k.append([rope(kk[h * dh:(h + 1) * dh], length + j) for h in range(D.heads)])
                v.append([vv[h * dh:(h + 1) * dh] for h in range(D.heads)])
            ck, cv = self.context_kv(l, kcaches[l], vcaches[l], length)
            o = []
            for j in range(4):
                row = []
                for h in range(D.heads):
                    keys = [c[h] for c in ck] + [k[i][h] for i in range(j + 1)]
                    vals = [c[h] for c in cv] + [v[i][h] for i in range(j + 1)]
                    sc = [sum(a * b for a, b in zip(q[j][h], key)) / math.sqrt(D.head_dim)
                          for key in keys]
                    mx = max(sc)
                    w = [math.exp(s - mx) for s in sc]
                    tot = sum(w)
                    row += [sum(wi * val[t] for wi, val in zip(w, vals)) / tot
                            for t in range(D.head_dim)]
                o.append(row)
            for j in range(4):
                x[j] = [a + b for a, b in zip(x[j], mv(W[p + "wo"], o[j]))]
                c = rms(x[j], m[p + "ffn_norm"])
                hcur = [silu(gv) * uv for gv, uv in zip(mv(W[p + "w_gate"], c), mv(W[p + "w_up"], c))]
                x[j] = [a + b for a, b in zip(x[j], mv(W[p + "w_down"], hcur))]
        logits = [mv(self.head, rms(x[j], m["final_norm"])) for j in range(4)]
        return logits

    def ingest_one(self, taps_rows, next_ids, length, kcaches, vcaches):
        """Return new caches (python copies) after appending rows."""
        m, W = self.m, self.W
        kc = [c.copy() for c in kcaches]
        vc = [c.copy() for c in vcaches]
        for i, (tr, tok) in enumerate(zip(taps_rows, next_ids)):
            pos = length + i
            f = mv(W["fuse"], [bf16(b) for b in tr.reshape(-1)])
            c = mv(W["fc"], f + self.embed(tok))
            for l in range(D.layers):
                p = f"layers.{l}."
                a = rms(c, m[p + "attn_norm"])
                kk, vv = mv(W[p + "wk"], a), mv(W[p + "wv"], a)
                dh = D.head_dim
                for h in range(D.heads):
                    kr = rope(kk[h * dh:(h + 1) * dh], pos)
                    kc[l][h, pos % D.capacity] = [
                        int(torch.tensor(val, dtype=torch.float64).to(torch.bfloat16)
                            .view(torch.int16).item()) & 0xFFFF for val in kr]
                    vc[l][h, pos % D.capacity] = [
                        int(torch.tensor(val, dtype=torch.float64).to(torch.bfloat16)
                            .view(torch.int16).item()) & 0xFFFF for val in vv[h * dh:(h + 1) * dh]]
        return kc, vc


@pytest.fixture(scope="module")
def setup():
    mnp = synth.to_numpy_model(synth.make_model(D, "C"))
    return mnp, oracle.OracleModel(mnp), Brute(mnp)


@pytest.mark.parametrize("length", [0, 5, 45])
def test_round_matches_brute_force(setup, length):
    mnp, M, brute = setup
    cfg = dict(name="bf", streams=1, lens=("const", length), model="C", ingest=0)
    inp = synth.to_numpy_inputs(synth.make_inputs(cfg, D, vocab=torch.from_numpy(mnp["vocab"]),
                                                  poison=True))
    logits, ids = oracle.oracle_round(M, inp)
    want = np.array(brute.round_one(inp["taps"][0], inp["anchor"][0], inp["pred"][0], length,
                                    [k[0] for k in inp["k"]], [v[0] for v in inp["v"]]))
    assert np.allclose(logits[0], want, rtol=1e-10, atol=1e-12)


def test_ingest_matches_brute_force(setup):
    mnp, M, brute = setup
    cfg = dict(name="bfi", streams=1, lens=("const", 30), model="C", ingest=3)
    inp = synth.to_numpy_inputs(synth.make_inputs(cfg, D, vocab=torch.from_numpy(mnp["vocab"]),
                                                  poison=True))
    after = oracle.oracle_ingest(M, inp)
    kc, vc = brute.ingest_one(inp["ingest_taps"][0], inp["ingest_ids"][0], 30,
                              [k[0] for k in inp["k"]], [v[0] for v in inp["v"]])
    for l in range(D.layers):
        # bf16 codes may differ by one ulp only where fp64 sums of different
        # order straddle a rounding boundary
        dk = np.abs(after["k"][l][0].astype(np.int64) - kc[l].astype(np.int64))
        dv = np.abs(after["v"][l][0].astype(np.int64) - vc[l].astype(np.int64))
        assert dk.max() <= 1 and dv.max() <= 1
        assert (dk > 0).mean() < 1e-3 and (dv > 0).mean() < 1e-3
    logits, _ = oracle.oracle_round(M, after)
    want = np.array(brute.round_one(inp["taps"][0], inp["anchor"][0], inp["pred"][0], 33, kc, vc))
    assert np.allclose(logits[0], want, rtol=1e-6, atol=1e-8)


def test_depth_two_matches_brute_force(setup):
    """Two rounds in a row (model card, Architecture, Serving; Predecessor
    head: at serving a row's predecessor is the drafter's own previous draft):
    the brute-force round run again with its own first-round drafts as
    predecessors."""
    mnp, M, brute = setup
    length = 20
    cfg = dict(name="bfd", streams=1, lens=("const", length), model="C", ingest=0)
    inp = synth.to_numpy_inputs(synth.make_inputs(cfg, D, vocab=torch.from_numpy(mnp["vocab"]),
                                                  poison=True))
    logits, ids = oracle.oracle_round_depth(M, inp, 2)
    kc, vc = [k[0] for k in inp["k"]], [v[0] for v in inp["v"]]
    first = brute.round_one(inp["taps"][0], inp["anchor"][0], inp["pred"][0], length, kc, vc)
    # each row's draft: the vocabulary entry at its first maximum
    drafts = []
    for row in first:
        best = 0
        for i in range(1, len(row)):
            if row[i] > row[best]:
                best = i
        drafts.append(int(mnp["vocab"][best]))
    second = np.array(brute.round_one(inp["taps"][0], inp["anchor"][0], drafts[:3], length, kc, vc))
    assert np.allclose(logits[0], second, rtol=1e-10, atol=1e-12)
    # row 0 never reads a predecessor: the same in both rounds
    assert np.allclose(logits[0][0], np.array(first[0]), rtol=1e-10, atol=1e-12)
    # the predecessors did change (else the test would not see the chaining)
    assert list(drafts[:3]) != [int(t) for t in inp["pred"][0]]
