"""GPU parity of the bf16 and block-FP8 head slices (the model card
"Kolibri-1 block drafter", section Use: the head slice can be bf16, FP8 or
NVFP4; Serving: the NVFP4 head keeps the drafts at a quarter of the bf16
bytes).

Up to 4 streams these heads run in the small-batch path's head phase (per
phase launches, path 2, and the persistent kernel, path 3), above 4 in the
general path's tiled head kernel. For bf16 each f16 activation is split
exactly into two bf16 terms for the bf16 matrix cores; for FP8 e4m3 is
decoded exactly to f16 and each 64-input block's product is scaled by its
row's scale. Acceptance as for every round: relative
L2 of the logits <= 1e-2 and ids equal wherever the oracle's top-1/top-2 gap
exceeds 1e-2.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from block_draft_model_amd import kdraft
from gpu_common import Harness, compare, log, require_gpu

pytestmark = pytest.mark.gpu

C = synth.CONFIGS


@pytest.fixture(scope="module", params=["bf16", "fp8"])
def hbC(request):
    require_gpu()
    return Harness("C", max_streams=256, head=request.param)


@pytest.mark.parametrize("path", [1, 2, 3])
def test_bf16_head_b4(hbC, path):
    inp = hbC.inputs(C[1])
    hbC.drafter.debug_set_path(path)
    try:
        lg, ids = hbC.run(inp)
        assert hbC.drafter.last_path() == path
    finally:
        hbC.drafter.debug_set_path(0)
    ref, rid = oracle.oracle_round(hbC.oracle, synth.to_numpy_inputs(inp))
    compare(lg, ids, ref, rid, hbC.oracle.vocab, f"{hbC.head} head B4 path {path}")


def test_small_path_heads_agree_bitwise_and_per_stream(hbC):
    """The two small-batch forms run the same head phase: identical logits;
    and a stream drafted alone equals the same stream in a batch of 4."""
    inp = hbC.inputs(C[1], base=23)
    out = {}
    for path in (2, 3):
        hbC.drafter.debug_set_path(path)
        try:
            out[path] = hbC.run(inp)
        finally:
            hbC.drafter.debug_set_path(0)
    assert np.array_equal(out[2][0], out[3][0]) and np.array_equal(out[2][1], out[3][1])
    one = {k: (v[1:2] if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    one["k"] = [t[1:2] for t in inp["k"]]
    one["v"] = [t[1:2] for t in inp["v"]]
    one["streams"] = 1
    lg1, ids1 = hbC.run(one)
    assert np.array_equal(lg1[0], out[2][0][1]) and np.array_equal(ids1[0], out[2][1][1])


def test_bf16_head_b1_and_edges(hbC):
    lens = [0, 1, 129, 2048, 6000]
    cfg = dict(name=f"{hbC.head} head edges", streams=len(lens), lens=("const", 0), model="C", ingest=0)
    inp = hbC.inputs(cfg, base=18, lens_override=lens)
    lg, ids = hbC.run(inp)
    ref, rid = oracle.oracle_round(hbC.oracle, synth.to_numpy_inputs(inp))
    compare(lg, ids, ref, rid, hbC.oracle.vocab, f"{hbC.head} head edges")
    one = hbC.inputs(C[0])
    lg, ids = hbC.run(one)
    ref, rid = oracle.oracle_round(hbC.oracle, synth.to_numpy_inputs(one))
    compare(lg, ids, ref, rid, hbC.oracle.vocab, f"{hbC.head} head B1")


def test_bf16_head_b16_ragged(hbC):
    inp = hbC.inputs(C[2])
    lg, ids = hbC.run(inp)
    ref, rid = oracle.oracle_round(hbC.oracle, synth.to_numpy_inputs(inp))
    compare(lg, ids, ref, rid, hbC.oracle.vocab, f"{hbC.head} head B16-ragged")


def test_bf16_head_b256_sampled(hbC):
    inp = hbC.inputs(C[4])
    lg, ids = hbC.run(inp)
    sample = [0, 5, 99, 200, 255]
    ref, rid = oracle.oracle_round(hbC.oracle, synth.to_numpy_inputs(inp, streams=sample))
    compare(lg[sample], ids[sample], ref, rid, hbC.oracle.vocab, f"{hbC.head} head B256 (sampled)")
    assert np.all(np.isin(ids, hbC.oracle.vocab))


def test_bf16_head_with_a_4bit_cache_and_depth(hbC):
    cfg = dict(name=f"{hbC.head} head int4", streams=6, lens=("uniform", 10, 3000), model="C", ingest=0)
    inp = hbC.inputs(cfg, base=19, kv="int4")
    B = inp["streams"]
    ids = torch.full((B, 4), -7, dtype=torch.int32, device="cuda")
    lg = torch.full((B, 4, synth.FULL.draft_vocab), float("nan"), device="cuda")
    hbC.drafter.round_depth(2, B, inp["taps"], inp["anchor"], inp["pred"], Harness.kv(inp),
                            inp["lens"], ids, lg)
    torch.cuda.synchronize()
    # round 1 alone, against the oracle's round 1
    lg1, ids1 = hbC.run(inp)
    inp_np = synth.to_numpy_inputs(inp)
    ref1, rid1 = oracle.oracle_round(hbC.oracle, inp_np)
    compare(lg1, ids1, ref1, rid1, hbC.oracle.vocab, f"{hbC.head} head, 4-bit cache, round 1")
    # round 2 against the oracle's own two-round chain, on the streams whose
    # round-1 drafts equal the oracle's (a near-tie draft on either side
    # changes the next round's predecessors)
    ref, rid = oracle.oracle_round_depth(hbC.oracle, inp_np, 2)
    same = np.all(ids1[:, :3] == rid1[:, :3], axis=1)
    assert same.any()
    compare(lg.cpu().numpy().astype(np.float64)[same], ids.cpu().numpy()[same], ref[same], rid[same],
            hbC.oracle.vocab, f"{hbC.head} head, 4-bit cache, depth 2")


def test_bf16_head_weight_errors():
    require_gpu()
    m = synth.make_model(synth.FULL, "A", device="cuda", head="bf16")
    d = kdraft.Drafter(max_streams=4, head_quant=kdraft.KD_QUANT_BF16)
    bad = dict(m)
    hb = m["head_bf16"].clone()
    hb[7, 3] = float("inf")
    bad["head_bf16"] = hb
    with pytest.raises(kdraft.KDraftError):
        d.load_weights(bad)
    none = dict(m)
    none["head_bf16"] = None
    with pytest.raises(kdraft.KDraftError):
        d.load_weights(none)
    d.load_weights(m)
    d.close()
