"""GPU parity of the NVFP4 and bf16 body weights (the model card "Kolibri-1
block drafter", section Use: the block body can be served in bf16, FP8 or
NVFP4; FP8 is the serving default).

These bodies run the general path at every batch size. NVFP4 codes times
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

import oracle
import synth
from gpu_common import Harness, compare, log, require_gpu

pytestmark = pytest.mark.gpu

C = synth.CONFIGS


@pytest.fixture(scope="module", params=["nvfp4", "bf16"])
def hb(request):
    require_gpu()
    return Harness("C", max_streams=256, body=request.param)


def test_body_b4_and_b1(hb):
    for cfg in (C[1], C[0]):
        inp = hb.inputs(cfg)
        lg, ids = hb.run(inp)
        assert hb.drafter.last_path() == 1
        ref, rid = oracle.oracle_round(hb.oracle, synth.to_numpy_inputs(inp))
        compare(lg, ids, ref, rid, hb.oracle.vocab, f"{hb.body} body {cfg['name']}")


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
