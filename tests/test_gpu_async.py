"""The ABI's asynchrony and input-checking conventions, on the GPU.

- kd_round enqueues and returns: with a long spin kernel queued ahead of it on
  the context's stream, the stream is still busy when kd_round returns, on the
  small-batch and the general path, also when the caller alternates between
  two buffer sets (the small path stages its argument blocks; the general path
  keeps a graph per buffer set). Results are bit-identical to single-buffer
  runs.
- token ids outside the table (the -1 / -2 sentinels a previous round may have
  written, or any other bad id) never index the embedding table: the rows that
  read them get out_ids -1 and the other rows are unchanged.
"""
import numpy as np
import pytest
import torch

import synth
from block_draft_model_amd import kdraft
from gpu_common import Harness, log, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hC():
    require_gpu()
    return Harness("C", max_streams=8)


def _buffers(h, inp):
    B = inp["streams"]
    ids = torch.full((B, 4), -7, dtype=torch.int32, device="cuda")
    lg = torch.full((B, 4, synth.FULL.draft_vocab), float("nan"), device="cuda")
    return ids, lg


def _enqueue(h, inp, ids, lg):
    h.drafter.round(inp["streams"], inp["taps"], inp["anchor"], inp["pred"], Harness.kv(inp),
                    inp["lens"], ids, lg)


@pytest.mark.parametrize("streams", [2, 6])   # small-batch path, general path
def test_round_returns_before_the_device_finishes(hC, streams):
    sets = []
    for base in (61, 62):
        cfg = dict(name=f"async{base}", streams=streams, lens=("uniform", 100, 2048), model="C", ingest=0)
        inp = hC.inputs(cfg, base=base)
        ids, lg = _buffers(hC, inp)
        _enqueue(hC, inp, ids, lg)                # first call per set: uploads / captures
        torch.cuda.synchronize()
        sets.append((inp, ids.clone(), lg.clone(), ids, lg))
    st = torch.cuda.current_stream()
    for rep in range(3):
        for inp, ref_ids, ref_lg, ids, lg in sets:
            ids.fill_(-7)
            lg.fill_(float("nan"))
            torch.cuda._sleep(20_000_000)          # tens of ms of spinning ahead of the round
            _enqueue(hC, inp, ids, lg)
            busy = not st.query()
            log(f"B={streams} rep {rep}: stream busy right after kd_round returned: {busy}, "
                f"path {hC.drafter.last_path()}")
            assert busy
    torch.cuda.synchronize()
    for inp, ref_ids, ref_lg, ids, lg in sets:
        assert torch.equal(ids, ref_ids)
        assert torch.equal(lg.nan_to_num(), ref_lg.nan_to_num())
        assert not torch.isnan(lg).any()


@pytest.mark.parametrize("path", [1, 2, 3])
def test_out_of_range_ids_mark_rows_and_are_never_read(hC, path):
    cfg = dict(name="bad-ids", streams=4, lens=("uniform", 50, 2048), model="C", ingest=0)
    inp = hC.inputs(cfg, base=67)
    V = synth.FULL.full_vocab
    hC.drafter.debug_set_path(path)
    try:
        good_lg, good_ids = hC.run(inp)
        bad = dict(inp)
        anchor = inp["anchor"].clone()
        pred = inp["pred"].clone()
        anchor[1] = -2                 # stream 1: the anchor (every row reads it)
        pred[2, 1] = -1                # stream 2: the predecessor of row 2 (rows 2, 3 read it)
        pred[3, 2] = V                 # stream 3: one past the table (row 3 reads it)
        bad["anchor"], bad["pred"] = anchor, pred
        lg, ids = hC.run(bad)
        assert hC.drafter.last_path() == path
    finally:
        hC.drafter.debug_set_path(0)
    want = good_ids.copy()
    want[1, :] = -1
    want[2, 2:] = -1
    want[3, 3] = -1
    log(f"path {path}: ids with bad inputs {ids.tolist()}")
    assert np.array_equal(ids, want)
    # stream 0 reads no bad id: bit-identical; rows before the bad predecessor
    # read nothing that changed either
    assert np.array_equal(lg[0], good_lg[0])
    assert np.array_equal(lg[2, :2], good_lg[2, :2])
    assert np.array_equal(lg[3, :3], good_lg[3, :3])
    assert np.all(np.isfinite(lg))
