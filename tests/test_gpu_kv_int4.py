"""GPU parity of the rotated 4-bit context cache (the article "Serving
Kolibri-1 with a 4-bit KV cache", section What we do) against the oracle.

Rounds: the cache holds seeded codes and fp16 (scale, offset) pairs; the
library turns each query by R = H diag(s)/sqrt(128) and reads the codes
directly, the oracle decodes the codes exactly and turns the keys back by R^T.
Both compute the same scores, so the round's acceptance rule is the bf16
cache's (relative L2 of the logits <= 1e-2, ids equal wherever the oracle's
top-1/top-2 gap exceeds 1e-2).

Ingest: the library rotates and codes each new row in fp32 from its f16-input
projections; the oracle does the same in fp64 from exact ones. Codes can
differ by one step where a value lies within the projection error of a
rounding boundary, so the check is the quantiser's own bound, applied to the
library's output against the oracle's exact rotated rows: every decoded value
lies within half a code step (plus the fp16 rounding of the row's minimum and
scale, and the projection error) of the exact value.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from block_draft_model_amd import kdraft
from gpu_common import Harness, compare, log, require_gpu
from oracle import kv_int4

pytestmark = pytest.mark.gpu

C = synth.CONFIGS


@pytest.fixture(scope="module")
def hA():
    require_gpu()
    return Harness("A")


@pytest.fixture(scope="module")
def hC():
    require_gpu()
    return Harness("C", max_streams=16)


def test_int4_round_context_length_edges(hC):
    # empty context, one row, 16-key block and 128-key boundaries, the full
    # window, and a context past the ring's capacity
    lens = [0, 1, 15, 16, 17, 129, 2047, 2048, 6000]
    cfg = dict(name="int4 edges", streams=len(lens), lens=("const", 0), model="C", ingest=0)
    inp = hC.inputs(cfg, base=12, lens_override=lens, kv="int4")
    log("int4 edges", lens)
    lg, ids = hC.run(inp)
    assert hC.drafter.last_path() == 1
    ref, rid = oracle.oracle_round(hC.oracle, synth.to_numpy_inputs(inp))
    compare(lg, ids, ref, rid, hC.oracle.vocab, "int4 length edges")


@pytest.mark.parametrize("path", [1, 2, 3])
def test_int4_small_batches(hC, path):
    """Up to 4 streams the 4-bit cache runs in the small-batch path's
    attention phase (path 2 per-phase launches, path 3 the persistent
    kernel): context-length edges (empty, one row, 16-key and 128-key
    boundaries, the full window, past the ring's capacity) and B = 1."""
    hC.drafter.debug_set_path(path)
    try:
        for i, lens in enumerate(([0, 1, 15, 16], [17, 129, 2047, 6000], [2048])):
            cfg = dict(name=f"int4 small {lens}", streams=len(lens), lens=("const", 0), model="C", ingest=0)
            inp = hC.inputs(cfg, base=40 + i, lens_override=lens, kv="int4")
            lg, ids = hC.run(inp)
            assert hC.drafter.last_path() == path
            ref, rid = oracle.oracle_round(hC.oracle, synth.to_numpy_inputs(inp))
            compare(lg, ids, ref, rid, hC.oracle.vocab, f"int4 path {path} lens {lens}")
    finally:
        hC.drafter.debug_set_path(0)


def test_int4_small_path_bitwise(hC):
    """Paths 2 and 3 run the same phase code (identical logits); a stream
    alone equals the same stream in a batch of 4 (its chunk partials do not
    depend on the batch)."""
    cfg = dict(name="int4 inv", streams=4, lens=("uniform", 10, 2600), model="C", ingest=0)
    inp = hC.inputs(cfg, base=44, kv="int4")
    out = {}
    for path in (2, 3):
        hC.drafter.debug_set_path(path)
        try:
            out[path] = hC.run(inp)
        finally:
            hC.drafter.debug_set_path(0)
    assert np.array_equal(out[2][0], out[3][0]) and np.array_equal(out[2][1], out[3][1])
    for b in (0, 3):
        one = {k: (v[b:b + 1] if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        for key in ("k", "v", "k_so", "v_so"):
            one[key] = [t[b:b + 1] for t in inp[key]]
        one["streams"] = 1
        lg1, ids1 = hC.run(one)
        assert np.array_equal(lg1[0], out[2][0][b]) and np.array_equal(ids1[0], out[2][1][b])


def test_int4_round_b16_ragged(hC):
    inp = hC.inputs(C[2], kv="int4")
    log("int4 B16 lens", inp["lens"].cpu().numpy().tolist())
    lg, ids = hC.run(inp)
    ref, rid = oracle.oracle_round(hC.oracle, synth.to_numpy_inputs(inp))
    compare(lg, ids, ref, rid, hC.oracle.vocab, "int4 B16-ragged")


def test_int4_round_b256_sampled(hA):
    inp = hA.inputs(C[4], kv="int4")
    lg, ids = hA.run(inp)
    sample = [0, 1, 77, 128, 200, 255]
    ref, rid = oracle.oracle_round(hA.oracle, synth.to_numpy_inputs(inp, streams=sample))
    compare(lg[sample], ids[sample], ref, rid, hA.oracle.vocab, "int4 B256 (sampled)")
    assert np.all(ids >= 0) and np.all(np.isin(ids, hA.oracle.vocab))


def test_int4_deterministic(hC):
    cfg = dict(name="det", streams=4, lens=("uniform", 100, 3000), model="C", ingest=0)
    inp = hC.inputs(cfg, base=13, kv="int4")
    a, ia = hC.run(inp)
    b, ib = hC.run(inp)
    assert np.array_equal(a, b) and np.array_equal(ia, ib)


def test_int4_ingest_then_round_b64(hA):
    cfg = C[3]
    inp = hA.inputs(cfg, kv="int4")
    sample = [0, 21, 63]
    before = synth.to_numpy_inputs(inp, streams=sample)
    hA.ingest(inp)
    assert np.array_equal(inp["lens"].cpu().numpy(), np.full(64, 2048))
    after_gpu = synth.to_numpy_inputs(inp, streams=sample)
    after_ref, exact = oracle.oracle_ingest(hA.oracle, before, return_exact=True)
    new = slice(2043, 2048)
    for l in range(4):
        for key, ex in (("k", exact[l][0]), ("v", exact[l][1])):
            x = ex.transpose(0, 2, 1, 3)                                   # [s][h][n][d]
            y = kv_int4.decode_int4(after_gpu[key][l][:, :, new], after_gpu[key + "_so"][l][:, :, new])
            sc = kv_int4.decode_f16(after_gpu[key + "_so"][l][:, :, new, 0])[..., None]
            rms = np.sqrt(np.mean(x * x, axis=-1, keepdims=True))
            amax = np.abs(x).max(axis=-1, keepdims=True)
            # half a step, the fp16 rounding of the row's minimum and scale
            # (at most 2^-10 of its largest value), and 2^-7 of the row's RMS
            # for the f16-input projections (measured errors stay near 2^-11)
            bound = 0.5 * sc + 2.0 ** -10 * amax + 2.0 ** -7 * rms
            err = np.abs(y - x)
            same = np.mean(after_gpu[key][l][:, :, new] == after_ref[key][l][:, :, new])
            log(f"int4 ingest layer {l} {key}: max err / step {float((err / sc).max()):.3f}, "
                f"beyond the bound {int((err > bound).sum())}/{err.size}, code bytes equal {same:.4f}")
            assert not (err > bound).any(), (l, key)
            assert same > 0.9, (l, key, same)
        # the rows before the new ones are untouched
        assert np.array_equal(after_gpu["k"][l][:, :, :2043], before["k"][l][:, :, :2043])
        assert np.array_equal(after_gpu["v_so"][l][:, :, :2043], before["v_so"][l][:, :, :2043])
    lg, ids = hA.run(inp)
    ref, rid = oracle.oracle_round(hA.oracle, after_ref)
    compare(lg[sample], ids[sample], ref, rid, hA.oracle.vocab, "int4 B64 after ingest (sampled)")


def test_int4_argument_errors(hC):
    cfg = dict(name="err", streams=2, lens=("const", 10), model="C", ingest=0)
    inp = hC.inputs(cfg, base=14, kv="int4")
    ids = torch.zeros((2, 4), dtype=torch.int32, device="cuda")
    kv = Harness.kv(inp)
    kv.format = 7
    with pytest.raises(kdraft.KDraftError):
        hC.drafter.round(2, inp["taps"], inp["anchor"], inp["pred"], kv, inp["lens"], ids)
    kv = Harness.kv(inp)
    kv.k_so[2] = None
    with pytest.raises(kdraft.KDraftError):
        hC.drafter.round(2, inp["taps"], inp["anchor"], inp["pred"], kv, inp["lens"], ids)
    kv = Harness.kv(inp)
    kv.v_so[1] = kv.v_so[1] + 2
    with pytest.raises(kdraft.KDraftError):
        hC.drafter.round(2, inp["taps"], inp["anchor"], inp["pred"], kv, inp["lens"], ids)


def _slot_major(inp):
    """The same cache stored slot-major ([B][capacity][heads][...] memory,
    viewed as [B][heads][capacity][...]): the row strides become
    (capacity * heads, 1, heads) instead of (heads * capacity, capacity, 1)."""
    out = dict(inp)
    for key in ("k", "v", "k_so", "v_so"):
        out[key] = [t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in inp[key]]
    return out


def test_int4_round_slot_major_layout(hC):
    cfg = dict(name="int4 strides", streams=5, lens=("uniform", 1, 5000), model="C", ingest=0)
    inp = hC.inputs(cfg, base=15, kv="int4")
    alt = _slot_major(inp)
    kv = Harness.kv(alt)
    assert (kv.stride_stream, kv.stride_head, kv.stride_slot) == (2048 * 20, 1, 20)
    a, ia = hC.run(inp)
    b, ib = hC.run(alt)
    # the same codes through other strides: the same round, bit for bit
    assert np.array_equal(a, b) and np.array_equal(ia, ib)
    ref, rid = oracle.oracle_round(hC.oracle, synth.to_numpy_inputs(alt))
    compare(b, ib, ref, rid, hC.oracle.vocab, "int4 slot-major layout")


def test_int4_depth_two_rounds(hC):
    cfg = dict(name="int4 depth", streams=6, lens=("uniform", 30, 2500), model="C", ingest=0)
    inp = hC.inputs(cfg, base=16, kv="int4")
    B = inp["streams"]
    kv = Harness.kv(inp)
    ids = torch.full((B, 4), -7, dtype=torch.int32, device="cuda")
    lg = torch.full((B, 4, synth.FULL.draft_vocab), float("nan"), device="cuda")
    hC.drafter.round_depth(2, B, inp["taps"], inp["anchor"], inp["pred"], kv, inp["lens"], ids, lg)
    torch.cuda.synchronize()
    lg1, ids1 = hC.run(inp)
    inp_np = synth.to_numpy_inputs(inp)
    ref1, rid1 = oracle.oracle_round(hC.oracle, inp_np)
    compare(lg1, ids1, ref1, rid1, hC.oracle.vocab, "int4 round 1")
    # round 2 on the streams whose round-1 drafts equal the oracle's: a
    # near-tie draft on either side changes the next round's predecessors
    ref, rid = oracle.oracle_round_depth(hC.oracle, inp_np, 2)
    same = np.all(ids1[:, :3] == rid1[:, :3], axis=1)
    assert same.any()
    compare(lg.cpu().numpy().astype(np.float64)[same], ids.cpu().numpy()[same], ref[same], rid[same],
            hC.oracle.vocab, "int4 depth 2")


def test_int4_ingest_wraps_the_ring(hC):
    # new rows past the ring's end land at slots 0, 1, ...; an empty context
    # and a long one (positions far past the capacity) as well
    lens = [2046, 4095, 0, 9000]
    cfg = dict(name="int4 ingest wrap", streams=4, lens=("const", 0), model="C", ingest=5)
    inp = hC.inputs(cfg, base=17, lens_override=lens, kv="int4")
    before = synth.to_numpy_inputs(inp)
    hC.ingest(inp)
    assert np.array_equal(inp["lens"].cpu().numpy(), np.array(lens) + 5)
    after_gpu = synth.to_numpy_inputs(inp)
    after_ref, exact = oracle.oracle_ingest(hC.oracle, before, return_exact=True)
    for l in range(4):
        for key, ex in (("k", exact[l][0]), ("v", exact[l][1])):
            for b, L in enumerate(lens):
                slots = [(L + i) % 2048 for i in range(5)]
                x = ex[b].transpose(1, 0, 2)                             # [h][n][d]
                y = kv_int4.decode_int4(after_gpu[key][l][b][:, slots], after_gpu[key + "_so"][l][b][:, slots])
                sc = kv_int4.decode_f16(after_gpu[key + "_so"][l][b][:, slots, 0])[..., None]
                rms = np.sqrt(np.mean(x * x, axis=-1, keepdims=True))
                amax = np.abs(x).max(axis=-1, keepdims=True)
                bound = 0.5 * sc + 2.0 ** -10 * amax + 2.0 ** -7 * rms
                assert not (np.abs(y - x) > bound).any(), (l, key, b)
    # the round on each side's own cache: the library's codes may differ by
    # one step from the oracle's where the projection error crosses a
    # rounding boundary (checked above). Over a full window those few steps
    # move the logits by ~1e-3; the stream whose whole context is the 5 new
    # rows sees each such step at full weight, so it is checked for valid
    # output only.
    lg, ids = hC.run(inp)
    ref, rid = oracle.oracle_round(hC.oracle, after_ref)
    rel = (np.linalg.norm(lg - ref, axis=-1) / np.linalg.norm(ref, axis=-1)).max(axis=-1)
    log("int4 round after a wrapping ingest, max rel L2 per stream", rel.tolist())
    full = [0, 1, 3]
    compare(lg[full], ids[full], ref[full], rid[full], hC.oracle.vocab,
            "int4 round after a wrapping ingest")
    assert np.all(np.isfinite(lg[2])) and np.all(np.isin(ids[2], hC.oracle.vocab))
