"""GPU parity of the NVFP4 and bf16 body weights (the model card "Kolibri-1
block drafter", section Use: the block body can be served in bf16, FP8 or
NVFP4; FP8 is the serving default).

Up to 4 streams these bodies run in the small-batch path's projection units
(per-phase launches, path 2, and the persistent kernel, path 3), above 4 in
the general path's tiled kernels. NVFP4 codes times
their e4m3 block scale decode exactly to f16 for the f16 matrix cores, and
each matrix's fp32 tensor scale multiplies the fp32 partial sums (the
predecessor adapter joins two matrices with their own tensor scales along
the inputs). bf16 weights meet each f16 activation split exactly into two
bf16 terms on the bf16 matrix cores. Acceptance as for every round:
relative L2 of the logits <= 1e-2 and ids equal wherever the oracle's
top-1/top-2 gap exceeds 1e-2. Model C (adapters active, random gains), so
every matrix and every gain contributes.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import Harness, compare, log, require_gpu

pytestmark = pytest.mark.gpu

C = synth.CONFIGS


@pytest.fixture(scope="module", params=["nvfp4", "bf16"])
def hb(request):
    require_gpu()
    return Harness("C", max_streams=256, body=request.param)


@pytest.mark.parametrize("path", [1, 2, 3])
def test_body_b4_and_b1(hb, path):
    hb.drafter.debug_set_path(path)
    try:
        for cfg in (C[1], C[0]):
            inp = hb.inputs(cfg)
            lg, ids = hb.run(inp)
            assert hb.drafter.last_path() == path
            ref, rid = oracle.oracle_round(hb.oracle, synth.to_numpy_inputs(inp))
            compare(lg, ids, ref, rid, hb.oracle.vocab, f"{hb.body} body {cfg['name']} path {path}")
    finally:
        hb.drafter.debug_set_path(0)


def test_small_path_bodies_agree_bitwise_and_per_stream(hb):
    """Paths 2 and 3 run the same phase code: identical logits; a stream
    drafted alone equals the same stream in a batch of 4; the small-path
    adapters with their gains (model C) on a ragged batch."""
    cfg = dict(name=f"{hb.body} small", streams=4, lens=("uniform", 10, 2600), model="C", ingest=0)
    inp = hb.inputs(cfg, base=29)
    out = {}
    for path in (2, 3):
        hb.drafter.debug_set_path(path)
        try:
            out[path] = hb.run(inp)
        finally:
            hb.drafter.debug_set_path(0)
    assert np.array_equal(out[2][0], out[3][0]) and np.array_equal(out[2][1], out[3][1])
    ref, rid = oracle.oracle_round(hb.oracle, synth.to_numpy_inputs(inp))
    compare(out[2][0], out[2][1], ref, rid, hb.oracle.vocab, f"{hb.body} body ragged B4, small path")
    one = {k: (v[2:3] if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    one["k"] = [t[2:3] for t in inp["k"]]
    one["v"] = [t[2:3] for t in inp["v"]]
    one["streams"] = 1
    lg1, ids1 = hb.run(one)
    assert np.array_equal(lg1[0], out[2][0][2]) and np.array_equal(ids1[0], out[2][1][2])


def test_body_context_edges(hb):
    lens = [0, 1, 129, 2048, 6000]
    cfg = dict(name=f"{hb.body} body edges", streams=len(lens), lens=("const", 0), model="C", ingest=0)
    inp = hb.inputs(cfg, base=19, lens_override=lens)
    lg, ids = hb.run(inp)
    ref, rid = oracle.oracle_round(hb.oracle, synth.to_numpy_inputs(inp))
    compare(lg, ids, ref, rid, hb.oracle.vocab, f"{hb.body} body edges")


def test_body_b16_ragged(hb):
    inp = hb.inputs(C[2])
    lg, ids = hb.run(inp)
    ref, rid = oracle.oracle_round(hb.oracle, synth.to_numpy_inputs(inp))
    compare(lg, ids, ref, rid, hb.oracle.vocab, f"{hb.body} body B16-ragged")


def test_body_b256_sampled(hb):
    # 1,024 block rows: the widest tiled projection kernel
    inp = hb.inputs(C[4])
    lg, ids = hb.run(inp)
    sample = [0, 1, 77, 128, 200, 255]
    ref, rid = oracle.oracle_round(hb.oracle, synth.to_numpy_inputs(inp, streams=sample))
    compare(lg[sample], ids[sample], ref, rid, hb.oracle.vocab, f"{hb.body} body B256 (sampled)")
    assert np.all(np.isin(ids, hb.oracle.vocab))


def test_body_ingest_then_round_b64_sampled(hb):
    # the ingest's fuse, fc and K/V projections read the same body matrices
    inp = hb.inputs(C[3])
    sample = [0, 33, 63]
    before = synth.to_numpy_inputs(inp, streams=sample)
    hb.ingest(inp)
    after_ref = oracle.oracle_ingest(hb.oracle, before)
    lg, ids = hb.run(inp)
    ref, rid = oracle.oracle_round(hb.oracle, after_ref)
    compare(lg[sample], ids[sample], ref, rid, hb.oracle.vocab, f"{hb.body} body B64 after ingest (sampled)")
    log(f"{hb.body} body: lengths after ingest {sorted(set(inp['lens'].cpu().tolist()))}")
