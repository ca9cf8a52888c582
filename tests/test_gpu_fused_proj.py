"""Fused q|k|v and gate|up epilogues of the general path (more than 32 block
rows), and the ingest's k|v projections of every layer in one launch (more
than 32 ingest rows), through the C ABI.

There the q|k|v and gate|up projections run in one split each and apply RoPE
and SwiGLU in the projection kernel. Checked against the fp64 oracle at the
smallest fused batch (9 streams, 36 block rows) and at a depth of two rounds,
against the split projections with separate epilogue kernels at several batch
sizes (partial 64-row blocks, both tile widths), and for run-to-run bit
equality. The ingest's projection stores the cache rows itself (bf16, or the
rotated 4-bit codes): checked against the oracle's exact K/V and against the
per-layer split projections with their store kernels.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import kv_int4
from block_draft_model_amd import kdraft
from gpu_common import GAP_MIN, Harness, compare, log, require_gpu

pytestmark = pytest.mark.gpu

# The two differ only in the order of the fp32 sums over the inputs (one split
# against several), which can move later f16 activation roundings by one ulp
# (2^-11 relative) here and there; the logits stay within 1e-3 of each other.
FUSED_VS_SEPARATE_REL_L2 = 1e-3


@pytest.fixture(scope="module")
def hF():
    require_gpu()
    return Harness("C", max_streams=100)


def _cfg(B, lo=0, hi=3000):
    return dict(name=f"fused-B{B}", streams=B, lens=("uniform", lo, hi), model="C", ingest=0)


def _run_depth(h, inp, depth):
    B = inp["streams"]
    kv = kdraft.kv_struct(inp["k"], inp["v"])
    ids = torch.full((B, 4), -7, dtype=torch.int32, device="cuda")
    lg = torch.full((B, 4, synth.FULL.draft_vocab), float("nan"), device="cuda")
    h.drafter.round_depth(depth, B, inp["taps"], inp["anchor"], inp["pred"], kv, inp["lens"], ids, lg)
    torch.cuda.synchronize()
    return lg.cpu().numpy().astype(np.float64), ids.cpu().numpy()


def test_fused_smallest_batch_against_oracle(hF):
    inp = hF.inputs(_cfg(9), base=61)
    lg, ids = hF.run(inp)
    assert hF.drafter.last_path() == 1
    ref, rid = oracle.oracle_round(hF.oracle, synth.to_numpy_inputs(inp))
    compare(lg, ids, ref, rid, hF.oracle.vocab, "fused B=9 (36 rows, spine on 27)")


@pytest.mark.parametrize("B", [9, 16, 37, 64, 100])
def test_fused_matches_separate_epilogues(hF, B):
    inp = hF.inputs(_cfg(B, 64, 2048), base=67 + B)
    lg_f, ids_f = hF.run(inp)
    hF.drafter.debug_set_fused(False)
    try:
        lg_s, ids_s = hF.run(inp)
    finally:
        hF.drafter.debug_set_fused(True)
    g = lg_f.reshape(-1, lg_f.shape[-1])
    s = lg_s.reshape(-1, lg_s.shape[-1])
    assert np.all(np.isfinite(g))
    rel = np.linalg.norm(g - s, axis=1) / np.linalg.norm(s, axis=1)
    gated = oracle.top2_gap(s) > GAP_MIN
    mism = int(np.sum((ids_f.reshape(-1) != ids_s.reshape(-1)) & gated))
    log(f"B={B}: fused vs separate max rel L2 {rel.max():.3e}, id mismatches on gated rows {mism}")
    assert rel.max() <= FUSED_VS_SEPARATE_REL_L2
    assert mism == 0


def test_fused_is_deterministic(hF):
    inp = hF.inputs(_cfg(37), base=71)
    a, ia = hF.run(inp)
    b, ib = hF.run(inp)
    assert np.array_equal(a, b) and np.array_equal(ia, ib)


def test_fused_depth_two_rounds(hF):
    inp = hF.inputs(_cfg(12, 100, 2500), base=73)
    lg1, ids1 = hF.run(inp)
    lg2, ids2 = _run_depth(hF, inp, 2)
    alt = dict(inp)
    alt["pred"] = torch.from_numpy(np.ascontiguousarray(ids1[:, :3])).to("cuda")
    lga, idsa = hF.run(alt)
    assert np.array_equal(lg2, lga) and np.array_equal(ids2, idsa)
    inp_np = synth.to_numpy_inputs(inp)
    _, o1 = oracle.oracle_round(hF.oracle, inp_np)
    ref, rid = oracle.oracle_round_depth(hF.oracle, inp_np, 2)
    same = np.all(ids1[:, :3] == o1[:, :3], axis=1)
    assert same.any()
    compare(lg2[same], ids2[same], ref[same], rid[same], hF.oracle.vocab, "fused depth 2, 12 streams")


# ---- the ingest's k|v projections of every layer in one launch ----

def _ingest_inputs(h, B, n, kv, base, lens=None):
    cfg = dict(name=f"ingest-B{B}x{n}", streams=B, lens=("uniform", 0, 5000), model="C", ingest=n)
    return h.inputs(cfg, base=base, kv=kv, lens_override=lens)


def _clone(inp):
    out = dict(inp)
    for key in ("k", "v", "k_so", "v_so"):
        if key in inp:
            out[key] = [t.clone() for t in inp[key]]
    out["lens"] = inp["lens"].clone()
    return out


def _written(inp_np, lens0, n, key, l):
    """The new rows of layer l ([B][heads][n][...]) at their ring slots."""
    cap = inp_np[key][l].shape[2]
    return np.stack([inp_np[key][l][b][:, [(int(L) + i) % cap for i in range(n)]]
                     for b, L in enumerate(lens0)])


def _decoded(inp_np, lens0, n, key, l, int4):
    x = _written(inp_np, lens0, n, key, l)
    if not int4:
        return oracle.decode_bf16(x), None
    so = _written(inp_np, lens0, n, key + "_so", l)
    return kv_int4.decode_int4(x, so), kv_int4.decode_f16(so[..., 0])[..., None]


@pytest.mark.parametrize("kv", ["bf16", "int4"])
def test_fused_ingest_against_oracle(hF, kv):
    # 36 ingest rows (a partial 64-row block); slots past the ring's end, an
    # empty context and positions far past the capacity
    lens = [2046, 4095, 0, 9000, 100, 2047, 1, 2040, 500]
    n = 4
    inp = _ingest_inputs(hF, len(lens), n, kv, 83, lens)
    before = synth.to_numpy_inputs(inp)
    hF.ingest(inp)
    assert np.array_equal(inp["lens"].cpu().numpy(), np.array(lens) + n)
    after = synth.to_numpy_inputs(inp)
    after_ref, exact = oracle.oracle_ingest(hF.oracle, before, return_exact=True)
    for l in range(4):
        for key, ex in (("k", exact[l][0]), ("v", exact[l][1])):
            x = ex.transpose(0, 2, 1, 3)                                   # [b][h][n][d]
            y, sc = _decoded(after, lens, n, key, l, kv == "int4")
            rms = np.sqrt(np.mean(x * x, axis=-1, keepdims=True))
            if kv == "int4":
                # half a code step, the fp16 offset's rounding, and the f16
                # input rows' projection error (as for the split projections)
                bound = 0.5 * sc + 2.0 ** -10 * np.abs(x).max(axis=-1, keepdims=True) + 2.0 ** -7 * rms
            else:
                # one bf16 ulp plus 2^-8 of the head vector's RMS (the f16
                # input rows' projection error)
                bound = np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 1e-30))) - 7) + 2.0 ** -8 * rms
            off = np.abs(y - x) > bound
            log(f"fused ingest {kv} layer {l} {key}: beyond the bound {int(off.sum())}/{off.size}")
            assert not off.any(), (kv, l, key)
    lg, ids = hF.run(inp)
    ref, rid = oracle.oracle_round(hF.oracle, after_ref)
    full = [b for b, L in enumerate(lens) if L >= 2048]
    compare(lg[full], ids[full], ref[full], rid[full], hF.oracle.vocab, f"{kv} round after a fused ingest")
    assert np.all(np.isfinite(lg))


@pytest.mark.parametrize("kv,B,n", [("bf16", 9, 4), ("bf16", 64, 5), ("bf16", 90, 8),
                                    ("int4", 9, 4), ("int4", 64, 5)])
def test_fused_ingest_matches_separate(hF, kv, B, n):
    inp = _ingest_inputs(hF, B, n, kv, 89 + B)
    lens0 = inp["lens"].cpu().numpy().copy()
    sep = _clone(inp)
    hF.ingest(inp)
    hF.drafter.debug_set_fused(False)
    try:
        hF.ingest(sep)
    finally:
        hF.drafter.debug_set_fused(True)
    assert np.array_equal(inp["lens"].cpu().numpy(), sep["lens"].cpu().numpy())
    a, b = synth.to_numpy_inputs(inp), synth.to_numpy_inputs(sep)
    worst = 0.0
    for l in range(4):
        for key in ("k", "v"):
            ya, sca = _decoded(a, lens0, n, key, l, kv == "int4")
            yb, scb = _decoded(b, lens0, n, key, l, kv == "int4")
            rms = np.sqrt(np.mean(yb * yb, axis=-1, keepdims=True))
            # the two differ in the order of the fp32 sums over the inputs
            # (one split against several) and in the RoPE angle's sine and
            # cosine precision: a value may round to the neighbouring bf16
            # number, a 4-bit code to the neighbouring step
            if kv == "int4":
                bound = np.maximum(sca, scb) * 1.0 + 2.0 ** -9 * rms
            else:
                bound = np.exp2(np.floor(np.log2(np.maximum(np.abs(yb), 1e-30))) - 7) + 2.0 ** -10 * rms
            err = np.abs(ya - yb)
            assert np.all(np.isfinite(ya)) and not (err > bound).any(), (kv, B, n, l, key)
            worst = max(worst, float((err / rms).max()))
    log(f"fused vs separate ingest {kv} B={B} n={n}: max diff / head RMS {worst:.2e}")
