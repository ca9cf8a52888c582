"""GPU parity of libkdraft against the fp64 oracle, through the C ABI.

Every context row outside a stream's window holds NaN (bf16), so a read
outside the window shows up as a non-finite logit. Workloads: the five seeded
synthetic configurations (B = 1, 4, 16 ragged, 64 with ingest, 256 ragged; the
larger two checked on sampled streams) and edge cases of the context length.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from block_draft_model_amd import kdraft
from gpu_common import GAP_MIN, Harness, compare, log, require_gpu

pytestmark = pytest.mark.gpu

C = synth.CONFIGS


@pytest.fixture(scope="module")
def hA():
    require_gpu()
    return Harness("A")


@pytest.fixture(scope="module")
def hB():
    require_gpu()
    return Harness("B", max_streams=16)


@pytest.fixture(scope="module")
def hC():
    require_gpu()
    return Harness("C", max_streams=8)


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    lib.hipMemcpy.restype = ctypes.c_int
    return lib


def device_floats(ptr, n):
    out = np.empty(n, dtype=np.float32)
    assert _hip().hipMemcpy(out.ctypes.data, ptr, n * 4, 2) == 0   # device -> host
    return out


def test_probe_e4m3_decoder_is_exact():
    require_gpu()
    out = torch.zeros(256, dtype=torch.int16, device="cuda")
    kdraft.probe_decode_e4m3(out)
    got = out.cpu().numpy().view(np.uint16)
    exact = oracle.decode_e4m3(np.arange(256))
    fin = np.isfinite(exact)
    assert np.array_equal(got[fin], oracle.round_bf16(exact[fin]))   # exact in bf16
    assert np.all(np.isnan(oracle.decode_bf16(got[~fin])))


def test_probe_e4m3_f16_decoder_is_exact():
    require_gpu()
    out = torch.zeros(256, dtype=torch.int16, device="cuda")
    kdraft.probe_decode_e4m3_f16(out)
    got = out.cpu().numpy().view(np.float16).astype(np.float64)
    exact = oracle.decode_e4m3(np.arange(256))
    fin = np.isfinite(exact)
    assert np.array_equal(got[fin], exact[fin])                  # every finite code exactly
    assert np.all(np.isnan(got[~fin]))


def test_probe_nvfp4_decoder_is_exact():
    require_gpu()
    out = torch.zeros(4096, dtype=torch.int16, device="cuda")
    kdraft.probe_decode_nvfp4(out)
    got = out.cpu().numpy().view(np.float16).astype(np.float64).reshape(256, 16)
    exact = oracle.decode_e4m3(np.arange(256))[:, None] * oracle.decode_e2m1(np.arange(16))[None, :]
    fin = np.isfinite(exact)
    assert np.array_equal(got[fin], exact[fin])                  # e2m1 x e4m3 exactly in f16


PATHS = [1, 2, 3]   # general multi-kernel, small-batch phases, small-batch persistent


@pytest.mark.parametrize("path", PATHS)
def test_layer_by_layer_b1(hA, path):
    """Bisection aid: hidden states after 0..4 layers against the oracle."""
    inp = hA.inputs(C[0])
    inp_np = synth.to_numpy_inputs(inp)
    M = hA.oracle
    full_layers = M.layers
    hA.drafter.debug_set_path(path)
    try:
        for n in range(0, 5):
            hA.drafter.debug_set_layers(n)
            lg, ids = hA.run(inp)
            hid, fus = hA.drafter.debug_buffers()
            x_gpu = device_floats(hid, 4 * 2560).reshape(1, 4, 2560)
            M.layers = full_layers[:n]
            ref, rid, x_ref = oracle.oracle_round(M, inp_np, return_hidden=True)
            relx = np.linalg.norm(x_gpu - x_ref, axis=-1) / np.linalg.norm(x_ref, axis=-1)
            log(f"layers={n} hidden rel err per row {relx.ravel()}")
            if n == 0:
                f_gpu = device_floats(fus, 2560)
                f_ref = oracle.decode_bf16(inp_np["taps"]).reshape(1, -1) @ M.fuse.T
                log("fused state rel err", np.linalg.norm(f_gpu - f_ref) / np.linalg.norm(f_ref))
            assert relx.max() < 1e-3
            assert hA.drafter.last_path() == path
            compare(lg, ids, ref, rid, M.vocab, f"path {path} layers={n}")
    finally:
        M.layers = full_layers
        hA.drafter.debug_set_layers(-1)
        hA.drafter.debug_set_path(0)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("ci", [0, 1])
def test_round_parity_small_batches(hA, ci, path):
    inp = hA.inputs(C[ci])
    hA.drafter.debug_set_path(path)
    try:
        lg, ids = hA.run(inp)
        assert hA.drafter.last_path() == path
    finally:
        hA.drafter.debug_set_path(0)
    ref, rid = oracle.oracle_round(hA.oracle, synth.to_numpy_inputs(inp))
    compare(lg, ids, ref, rid, hA.oracle.vocab, f"{C[ci]['name']} path {path}")


@pytest.mark.parametrize("path", [2, 3])
def test_small_path_adapters_gains_and_edges(hC, path):
    """Active spine and predecessor adapters, random gains, and context
    lengths 0, 1, a chunk boundary + 1 and past the ring, on the <= 4-stream path."""
    lens = [0, 1, 129, 6000]
    cfg = dict(name="small-edges", streams=4, lens=("const", 0), model="C", ingest=0)
    inp = hC.inputs(cfg, base=23, lens_override=lens)
    hC.drafter.debug_set_path(path)
    try:
        lg, ids = hC.run(inp)
        assert hC.drafter.last_path() == path
    finally:
        hC.drafter.debug_set_path(0)
    ref, rid = oracle.oracle_round(hC.oracle, synth.to_numpy_inputs(inp))
    compare(lg, ids, ref, rid, hC.oracle.vocab, f"model C small path {path}")


@pytest.mark.parametrize("path", [2, 3])
@pytest.mark.parametrize("lens", [[700], [1, 300], [0, 0, 5, 128], [0, 0]])
def test_small_path_fewer_chunks_than_workgroups(hC, path, lens):
    """Short contexts: fewer 128-row chunks in the round than workgroups, so
    some workgroups get no attention work and every chunk is its own segment
    (and no context at all: block-only attention)."""
    cfg = dict(name="short", streams=len(lens), lens=("const", 0), model="C", ingest=0)
    inp = hC.inputs(cfg, base=37, lens_override=lens)
    hC.drafter.debug_set_path(path)
    try:
        lg, ids = hC.run(inp)
        assert hC.drafter.last_path() == path
    finally:
        hC.drafter.debug_set_path(0)
    ref, rid = oracle.oracle_round(hC.oracle, synth.to_numpy_inputs(inp))
    compare(lg, ids, ref, rid, hC.oracle.vocab, f"short contexts {lens} path {path}")


def test_small_paths_agree_bitwise_and_are_deterministic(hC):
    cfg = dict(name="agree", streams=3, lens=("uniform", 1, 3000), model="C", ingest=0)
    inp = hC.inputs(cfg, base=29)
    outs = []
    for path in (2, 3, 3, 2):
        hC.drafter.debug_set_path(path)
        outs.append(hC.run(inp))
    hC.drafter.debug_set_path(0)
    for lg, ids in outs[1:]:
        assert np.array_equal(lg, outs[0][0]) and np.array_equal(ids, outs[0][1])


@pytest.mark.parametrize("path", PATHS)
def test_small_path_stream_alone_equals_stream_in_batch(hC, path):
    # The model card's Serving section drafts every stream in one batched
    # pass; a stream's drafts must not depend on the batch around it. Every
    # attention chunk stores its own softmax partial and a stream's partials
    # are merged in chunk order, the projections compute every row on its
    # own, so a stream alone and in a batch agree bit for bit.
    cfg = dict(name="inv-small", streams=4, lens=("uniform", 10, 2048), model="C", ingest=0)
    inp = hC.inputs(cfg, base=31)
    hC.drafter.debug_set_path(path)
    try:
        batch, ib = hC.run(inp)
        assert hC.drafter.last_path() == path
        for b in range(4):
            one = {k: (v[b:b + 1] if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
            one["k"] = [t[b:b + 1] for t in inp["k"]]
            one["v"] = [t[b:b + 1] for t in inp["v"]]
            one["streams"] = 1
            alone, ia = hC.run(one)
            rel = np.linalg.norm(alone[0] - batch[b], axis=1) / np.linalg.norm(batch[b], axis=1)
            log(f"path {path} stream {b} alone vs in batch: max rel L2 {rel.max():.2e}")
            assert np.array_equal(alone[0], batch[b])
            assert np.array_equal(ia[0], ib[b])
    finally:
        hC.drafter.debug_set_path(0)


@pytest.mark.parametrize("path", [2, 3])
def test_small_path_full_batch_equals_streams_alone(hC, path):
    # 4 streams with full windows make 1,280 attention units, more than 4
    # per workgroup: one wave computes both halves of each chunk; a stream
    # alone (320 units) splits every chunk over a wave pair. A chunk's partial
    # is the same merge of its two half states either way, so the drafts
    # agree bit for bit. Positions past the ring's capacity wrap.
    lens = [2048, 2500, 4100, 9000]
    cfg = dict(name="inv-full", streams=4, lens=("const", 0), model="C", ingest=0)
    inp = hC.inputs(cfg, base=41, lens_override=lens)
    hC.drafter.debug_set_path(path)
    try:
        batch, ib = hC.run(inp)
        assert hC.drafter.last_path() == path
        for b in range(4):
            one = {k: (v[b:b + 1] if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
            one["k"] = [t[b:b + 1] for t in inp["k"]]
            one["v"] = [t[b:b + 1] for t in inp["v"]]
            one["streams"] = 1
            alone, ia = hC.run(one)
            rel = np.linalg.norm(alone[0] - batch[b], axis=1) / np.linalg.norm(batch[b], axis=1)
            log(f"path {path} full-window stream {b} alone vs in batch: max rel L2 {rel.max():.2e}")
            assert np.array_equal(alone[0], batch[b])
            assert np.array_equal(ia[0], ib[b])
    finally:
        hC.drafter.debug_set_path(0)
    ref, rid = oracle.oracle_round(hC.oracle, synth.to_numpy_inputs(inp))
    compare(batch, ib, ref, rid, hC.oracle.vocab, f"full windows path {path}")


def test_round_parity_adapters_and_gains_active(hC):
    cfg = dict(name="C-B5", streams=5, lens=("uniform", 0, 3000), model="C", ingest=0)
    inp = hC.inputs(cfg, base=7)
    lg, ids = hC.run(inp)
    ref, rid = oracle.oracle_round(hC.oracle, synth.to_numpy_inputs(inp))
    compare(lg, ids, ref, rid, hC.oracle.vocab, "model C, B=5")


def test_round_parity_b16_ragged(hB):
    inp = hB.inputs(C[2])
    lens = inp["lens"].cpu().numpy()
    log("B16 lens", lens.tolist())
    lg, ids = hB.run(inp)
    ref, rid = oracle.oracle_round(hB.oracle, synth.to_numpy_inputs(inp))
    compare(lg, ids, ref, rid, hB.oracle.vocab, C[2]["name"])


def test_context_length_edges(hC):
    # empty context, a single row, chunk boundaries, the full window, and
    # contexts past the ring's capacity (positions wrap, RoPE keeps counting)
    lens = [0, 1, 127, 128, 129, 2047, 2048, 6000]
    cfg = dict(name="edges", streams=len(lens), lens=("const", 0), model="C", ingest=0)
    inp = hC.inputs(cfg, base=11, lens_override=lens)
    lg, ids = hC.run(inp)
    ref, rid = oracle.oracle_round(hC.oracle, synth.to_numpy_inputs(inp))
    compare(lg, ids, ref, rid, hC.oracle.vocab, "length edges")


def test_ingest_then_round_b64(hA):
    cfg = C[3]
    inp = hA.inputs(cfg)
    sample = [0, 21, 63]
    before = synth.to_numpy_inputs(inp, streams=sample)
    hA.ingest(inp)
    assert np.array_equal(inp["lens"].cpu().numpy(), np.full(64, 2048))
    after_gpu = synth.to_numpy_inputs(inp, streams=sample)
    after_ref, exact = oracle.oracle_ingest(hA.oracle, before, return_exact=True)
    for l in range(4):
        for key, ex in (("k", exact[l][0]), ("v", exact[l][1])):
            g = oracle.decode_bf16(after_gpu[key][l][:, :, 2043:2048])   # [s][h][n][d]
            e = ex.transpose(0, 2, 1, 3)                                  # [s][h][n][d]
            # the normalised row enters the K/V projections as f16 (11
            # significant bits): each value carries an error of about 2^-12 of
            # its head vector's RMS (std over 2560 rounded inputs), which can
            # move it past a bf16 rounding boundary. Bound: one bf16 ulp of the
            # exact value plus 2^-8 of the head vector's RMS (over 10 std of
            # that error; a wrong input or weight gives errors of order the RMS)
            ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(e), 1e-30))) - 7)
            scale = np.sqrt(np.mean(e * e, axis=-1, keepdims=True))
            rel = np.abs(g - e) / np.maximum(np.abs(e), 1e-30)
            err = np.abs(g - e) / scale
            off = np.abs(g - e) > ulp + 2.0 ** -8 * scale
            log(f"ingest layer {l} {key}: max rel err {rel.max():.3e}, "
                f"max err / head RMS {err.max():.2e}, beyond the bound {int(off.sum())}/{off.size}, "
                f"codes differing from oracle {(after_gpu[key][l][:, :, 2043:2048] != after_ref[key][l][:, :, 2043:2048]).mean():.2e}")
            assert not off.any(), (l, key)
    lg, ids = hA.run(inp)
    ref, rid = oracle.oracle_round(hA.oracle, after_ref)
    compare(lg[sample], ids[sample], ref, rid, hA.oracle.vocab, "B64 after ingest (sampled)")


def test_round_parity_b256_sampled(hA):
    inp = hA.inputs(C[4])
    lg, ids = hA.run(inp)
    sample = [0, 1, 77, 128, 200, 255]
    ref, rid = oracle.oracle_round(hA.oracle, synth.to_numpy_inputs(inp, streams=sample))
    compare(lg[sample], ids[sample], ref, rid, hA.oracle.vocab, "B256 (sampled)")
    assert np.all(ids >= 0) and np.all(np.isin(ids, hA.oracle.vocab))


def test_round_parity_b100_partial_row_block(hA):
    """100 streams = 400 block rows: the projections take the widest tiled
    kernel (more than 256 rows), whose last 64-row block is a quarter full
    (rows 384..399 = streams 96..99). Sampled streams in the first and the
    partial block."""
    cfg = dict(name="B100", streams=100, lens=("uniform", 512, 2048), model="A", ingest=0)
    inp = hA.inputs(cfg, base=53)
    lg, ids = hA.run(inp)
    assert hA.drafter.last_path() == 1
    sample = [0, 37, 95, 96, 97, 99]
    ref, rid = oracle.oracle_round(hA.oracle, synth.to_numpy_inputs(inp, streams=sample))
    compare(lg[sample], ids[sample], ref, rid, hA.oracle.vocab, "B100 (sampled, partial row block)")
    assert np.all(np.isin(ids, hA.oracle.vocab))


@pytest.mark.parametrize("path", PATHS)
def test_deterministic_and_logits_optional(hC, path):
    cfg = dict(name="det", streams=3, lens=("uniform", 100, 2500), model="C", ingest=0)
    inp = hC.inputs(cfg, base=13)
    hC.drafter.debug_set_path(path)
    a, ia = hC.run(inp)
    b, ib = hC.run(inp)
    assert np.array_equal(a, b) and np.array_equal(ia, ib)
    _, ic = hC.run(inp, logits=False)
    hC.drafter.debug_set_path(0)
    assert np.array_equal(ia, ic)


def test_stream_alone_equals_stream_in_batch(hC):
    cfg = dict(name="inv", streams=4, lens=("uniform", 10, 2048), model="C", ingest=0)
    inp = hC.inputs(cfg, base=17)
    hC.drafter.debug_set_path(1)
    batch, ib = hC.run(inp)
    for b in range(4):
        one = {k: (v[b:b + 1] if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        one["k"] = [t[b:b + 1] for t in inp["k"]]
        one["v"] = [t[b:b + 1] for t in inp["v"]]
        one["streams"] = 1
        alone, ia = hC.run(one)
        assert np.array_equal(alone[0], batch[b]) and np.array_equal(ia[0], ib[b])
    hC.drafter.debug_set_path(0)


def _run_depth(h, inp, depth):
    B = inp["streams"]
    kv = kdraft.kv_struct(inp["k"], inp["v"])
    ids = torch.full((B, 4), -7, dtype=torch.int32, device="cuda")
    lg = torch.full((B, 4, synth.FULL.draft_vocab), float("nan"), device="cuda")
    h.drafter.round_depth(depth, B, inp["taps"], inp["anchor"], inp["pred"], kv, inp["lens"], ids, lg)
    torch.cuda.synchronize()
    return lg.cpu().numpy().astype(np.float64), ids.cpu().numpy()


@pytest.mark.parametrize("path", PATHS)
def test_depth_two_rounds(hC, path):
    """Two rounds in a row: the second takes the first's drafts as its
    predecessor ids on the device. It equals a round called with those drafts
    as pred_ids, and both rounds meet the acceptance rule against the oracle
    (round 2's reference is the oracle's own two-round chain; it is compared
    on the streams whose round-1 drafts equal the oracle's, since a near-tie
    draft of either side changes the next round's predecessors)."""
    cfg = dict(name="depth", streams=3, lens=("uniform", 50, 2500), model="C", ingest=0)
    inp = hC.inputs(cfg, base=37)
    hC.drafter.debug_set_path(path)
    try:
        lg1, ids1 = hC.run(inp)
        lg2, ids2 = _run_depth(hC, inp, 2)
        assert hC.drafter.last_path() == path
        alt = dict(inp)
        alt["pred"] = torch.from_numpy(np.ascontiguousarray(ids1[:, :3])).to("cuda")
        lga, idsa = hC.run(alt)
        lgd1, idsd1 = _run_depth(hC, inp, 1)
    finally:
        hC.drafter.debug_set_path(0)
    assert np.array_equal(lgd1, lg1) and np.array_equal(idsd1, ids1)   # depth 1 is kd_round
    assert np.array_equal(lg2, lga) and np.array_equal(ids2, idsa)
    assert np.array_equal(lg2[:, 0], lg1[:, 0])                      # row 0 reads no predecessor
    assert not np.array_equal(ids1[:, :3], inp["pred"].cpu().numpy())  # the predecessors changed
    assert not np.allclose(lg2[:, 1:], lg1[:, 1:], rtol=1e-3, atol=1e-3)  # and moved rows 1..3
    ref1, rid1 = oracle.oracle_round(hC.oracle, synth.to_numpy_inputs(inp))
    compare(lg1, ids1, ref1, rid1, hC.oracle.vocab, f"depth round 1 path {path}")
    ref2, rid2 = oracle.oracle_round_depth(hC.oracle, synth.to_numpy_inputs(inp), 2)
    same = np.all(ids1[:, :3] == rid1[:, :3], axis=1)
    assert same.any()
    compare(lg2[same], ids2[same], ref2[same], rid2[same], hC.oracle.vocab,
            f"depth round 2 path {path}")


def test_depth_general_path_batch(hB):
    # more than 4 streams: the general path chains the rounds inside one graph
    cfg = dict(name="depth-gen", streams=6, lens=("uniform", 200, 2048), model="B", ingest=0)
    inp = hB.inputs(cfg, base=41)
    lg1, ids1 = hB.run(inp)
    lg3, ids3 = _run_depth(hB, inp, 3)
    alt = dict(inp)
    alt["pred"] = torch.from_numpy(np.ascontiguousarray(ids1[:, :3])).to("cuda")
    lg2, ids2 = hB.run(alt)
    alt2 = dict(inp)
    alt2["pred"] = torch.from_numpy(np.ascontiguousarray(ids2[:, :3])).to("cuda")
    lga, idsa = hB.run(alt2)
    assert np.array_equal(lg3, lga) and np.array_equal(ids3, idsa)
    # the oracle's own three-round chain, on the streams whose first two
    # rounds drafted what the oracle's did
    inp_np = synth.to_numpy_inputs(inp)
    _, o1 = oracle.oracle_round(hB.oracle, inp_np)
    _, o2 = oracle.oracle_round_depth(hB.oracle, inp_np, 2)
    ref, rid = oracle.oracle_round_depth(hB.oracle, inp_np, 3)
    same = np.all(ids1[:, :3] == o1[:, :3], axis=1) & np.all(ids2[:, :3] == o2[:, :3], axis=1)
    assert same.any()
    compare(lg3[same], ids3[same], ref[same], rid[same], hB.oracle.vocab, "depth 3, 6 streams")


def test_depth_argument_errors(hC):
    cfg = dict(name="derr", streams=2, lens=("const", 5), model="C", ingest=0)
    inp = hC.inputs(cfg, base=43)
    for depth in (0, 9):
        with pytest.raises(kdraft.KDraftError) as e:
            _run_depth(hC, inp, depth)
        assert e.value.status == kdraft.KD_ERR_ARG


def test_gpu_argument_errors(hC):
    B = 2
    cfg = dict(name="err", streams=B, lens=("const", 5), model="C", ingest=0)
    inp = hC.inputs(cfg, base=19)
    kv = kdraft.kv_struct(inp["k"], inp["v"])
    ids = torch.empty(B, 4, dtype=torch.int32, device="cuda")
    with pytest.raises(kdraft.KDraftError) as e:
        hC.drafter.round(9, inp["taps"], inp["anchor"], inp["pred"], kv, inp["lens"], ids)
    assert e.value.status == kdraft.KD_ERR_ARG
    with pytest.raises(kdraft.KDraftError) as e:
        hC.drafter.round(B, None, inp["anchor"], inp["pred"], kv, inp["lens"], ids)
    assert e.value.status == kdraft.KD_ERR_ARG
    small = kdraft.kv_struct([t[:, :, :1024] for t in inp["k"]], [t[:, :, :1024] for t in inp["v"]])
    with pytest.raises(kdraft.KDraftError) as e:
        hC.drafter.round(B, inp["taps"], inp["anchor"], inp["pred"], small, inp["lens"], ids)
    assert e.value.status == kdraft.KD_ERR_ARG
    fresh = kdraft.Drafter(max_streams=2)
    with pytest.raises(kdraft.KDraftError) as e:
        fresh.round(B, inp["taps"], inp["anchor"], inp["pred"], kv, inp["lens"], ids)
    assert e.value.status == kdraft.KD_ERR_STATE
    fresh.close()
