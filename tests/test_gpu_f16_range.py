"""Activations beyond the f16 range. Matrix inputs are stored in f16; the
small-batch path stores the residual stream times its RMSNorm gain before
normalising (the norm needs every tile's sum of squares), so residual
components above 65,504 cannot be held there. Such a store saturates and
flags the round; the next call returns KD_ERR_RANGE (once: reading the flag
clears it). A path that never stores such a value keeps parity with the
oracle.

The model: model C with the mask row scaled to a standard deviation of 1e5,
which rows 1..3 of every block carry in their residual stream."""
import pytest
import torch

import oracle
import synth
from block_draft_model_amd import kdraft
from gpu_common import compare, log, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def big():
    require_gpu()
    m = synth.make_model(synth.FULL, "C", device="cuda")
    m["mask"] = m["mask"] * 5.0e6          # N(0, 0.02) -> N(0, 1e5)
    d = kdraft.Drafter(max_streams=8)
    d.load_weights(m)
    yield m, d, oracle.OracleModel(synth.to_numpy_model(m))
    d.close()


def _round(d, inp):
    B = inp["streams"]
    ids = torch.full((B, 4), -7, dtype=torch.int32, device="cuda")
    lg = torch.full((B, 4, synth.FULL.draft_vocab), float("nan"), device="cuda")
    d.round(B, inp["taps"], inp["anchor"], inp["pred"], kdraft.kv_struct(inp["k"], inp["v"]), inp["lens"], ids, lg)
    torch.cuda.synchronize()
    return lg.cpu().numpy(), ids.cpu().numpy()


def _next_call_status(d, inp):
    try:
        _round(d, inp)
        return kdraft.KD_OK
    except kdraft.KDraftError as e:
        return e.status


def _settled_round(d, inp):
    """A round that ran: a call that reports an earlier round's range flag
    enqueues nothing, so such a call is repeated (at most once)."""
    for _ in range(2):
        try:
            return _round(d, inp)
        except kdraft.KDraftError as e:
            assert e.status == kdraft.KD_ERR_RANGE, e
    raise AssertionError("a range report came twice in a row")


@pytest.mark.parametrize("path", [1, 2, 3])
def test_huge_residuals_keep_parity_or_report_the_range(big, path):
    m, d, M = big
    cfg = dict(name="range", streams=2, lens=("uniform", 300, 2048), model="C", ingest=0)
    inp = synth.make_inputs(cfg, synth.FULL, device="cuda", vocab=m["vocab"], base=71)
    d.debug_set_path(path)
    try:
        lg, ids = _settled_round(d, inp)
        status = _next_call_status(d, inp)   # reports the round above
        again = _next_call_status(d, inp)    # reports the round the call above enqueued, if any
        assert d.last_path() == path
    finally:
        d.debug_set_path(0)
    log(f"path {path}: next call {kdraft.status_string(status)}")
    assert status in (kdraft.KD_OK, kdraft.KD_ERR_RANGE)
    if path in (2, 3):
        # the gained residual is stored unnormalised in f16: saturated, reported
        assert status == kdraft.KD_ERR_RANGE
        # the failing call enqueued nothing, so nothing is reported for it
        assert again == kdraft.KD_OK
    if status == kdraft.KD_OK:
        ref, rid = oracle.oracle_round(M, synth.to_numpy_inputs(inp))
        compare(lg, ids, ref, rid, M.vocab, f"huge residuals, path {path}")
