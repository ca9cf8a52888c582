"""Round-level pins of the oracle (tiny model of the same structure).

What the model card ("Kolibri-1 block drafter", Architecture) fixes:
* the spine leaves row 0 untouched (Spine bullet);
* row 0 sees exactly what a chain drafter sees (Position 1 bullet): row 0 of a
  4-row block equals a 1-row block;
* the block is causal (Body bullet): no row depends on later rows' inputs;
* only the last 2,048 (here: window) context rows are attended (Body bullet);
* the head is the LM head restricted to the draft vocabulary (Output bullet);
* every stream is drafted in one batched pass (Serving): a stream's result
  does not depend on the batch around it.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth

D = synth.TINY
CFG = dict(name="tiny", streams=3, lens=("uniform", 1, 60), model="B", ingest=0)


@pytest.fixture(scope="module")
def models():
    out = {}
    for v in ("A", "B", "C"):
        m = synth.make_model(D, v)
        out[v] = (synth.to_numpy_model(m), oracle.OracleModel(synth.to_numpy_model(m)))
    return out


@pytest.fixture(scope="module")
def inputs(models):
    inp = synth.make_inputs(CFG, D, vocab=torch.from_numpy(models["B"][0]["vocab"]), poison=True)
    return synth.to_numpy_inputs(inp)


def test_outputs_are_finite_and_ids_in_vocab(models, inputs):
    for v in "ABC":
        logits, ids = oracle.oracle_round(models[v][1], inputs)
        assert logits.shape == (3, 4, D.draft_vocab)
        assert np.all(np.isfinite(logits))
        assert np.all(np.isin(ids, models[v][0]["vocab"]))
        # ids are the vocabulary entries at the first maximum
        assert np.array_equal(ids, models[v][0]["vocab"][np.argmax(logits, axis=-1)])


def test_spine_off_leaves_row0_unchanged(models, inputs):
    M = models["C"][1]
    on, _ = oracle.oracle_round(M, inputs)
    off, _ = oracle.oracle_round(M, inputs, spine=False)
    assert np.array_equal(on[:, 0], off[:, 0])
    assert not np.allclose(on[:, 1:], off[:, 1:])


def test_row0_is_the_chain_drafter_row(models, inputs):
    M = models["C"][1]
    full, _ = oracle.oracle_round(M, inputs)
    chain, _ = oracle.oracle_round(M, inputs, block=1)
    assert np.allclose(full[:, 0], chain[:, 0], rtol=1e-12, atol=1e-12)


def test_causal_in_block(models, inputs):
    M = models["B"][1]
    vocab = models["B"][0]["vocab"]
    base, _ = oracle.oracle_round(M, inputs)
    for j in range(3):                       # pred[j] feeds row j + 1
        alt = dict(inputs)
        alt["pred"] = inputs["pred"].copy()
        alt["pred"][:, j] = vocab[(np.searchsorted(vocab, alt["pred"][:, j]) + 7) % len(vocab)]
        got, _ = oracle.oracle_round(M, alt)
        assert np.array_equal(got[:, : j + 1], base[:, : j + 1])
        assert not np.allclose(got[:, j + 1], base[:, j + 1])


def test_zero_adapters_ignore_predecessors(models, inputs):
    M = models["A"][1]
    vocab = models["A"][0]["vocab"]
    base, _ = oracle.oracle_round(M, inputs)
    alt = dict(inputs)
    alt["pred"] = np.full_like(inputs["pred"], vocab[5])
    got, _ = oracle.oracle_round(M, alt)
    assert np.array_equal(got, base)


def test_anchor_feeds_row0(models, inputs):
    M = models["A"][1]
    vocab = models["A"][0]["vocab"]
    base, _ = oracle.oracle_round(M, inputs)
    alt = dict(inputs)
    alt["anchor"] = np.full_like(inputs["anchor"], vocab[11])
    got, _ = oracle.oracle_round(M, alt)
    assert not np.allclose(got[:, 0], base[:, 0])


def test_restricted_head_equals_gathered_full_head(models, inputs):
    mnp, M = models["C"]
    logits, _, x = oracle.oracle_round(M, inputs, return_hidden=True)
    table = torch.from_numpy(mnp["table"].view(np.int16)).view(torch.bfloat16).float()
    q4, s4, _ = synth.quant_nvfp4(table, g=mnp["head.g"])
    full = oracle.nvfp4(q4.numpy(), s4.numpy(), mnp["head.g"])
    z = oracle.rmsnorm(x, M.final_norm, D.rms_eps)
    assert np.allclose((z @ full.T)[..., mnp["vocab"]], logits, rtol=1e-12, atol=1e-12)


def test_stream_alone_equals_stream_in_batch(models, inputs):
    M = models["C"][1]
    batch, ids = oracle.oracle_round(M, inputs)
    for b in range(3):
        one = {k: (v[b:b + 1] if isinstance(v, np.ndarray) else v) for k, v in inputs.items()}
        one["k"] = [t[b:b + 1] for t in inputs["k"]]
        one["v"] = [t[b:b + 1] for t in inputs["v"]]
        one["streams"] = 1
        alone, ida = oracle.oracle_round(M, one)
        assert np.allclose(alone[0], batch[b], rtol=1e-12, atol=1e-12)


def test_window_keeps_only_the_last_rows(models):
    """A context longer than the window equals the same rows stored in a bigger
    ring where nothing else is visible, and rows outside the window (NaN) are
    never read."""
    mnp, M = models["B"]
    big = dataclasses.replace(D, capacity=64)
    cfg = dict(name="w", streams=1, lens=("const", 50), model="B", ingest=0)
    src = synth.to_numpy_inputs(synth.make_inputs(cfg, big, vocab=torch.from_numpy(mnp["vocab"])))
    # ring of capacity 32 = window: position p at slot p % 32
    small = dict(src)
    small["k"], small["v"] = [], []
    for l in range(D.layers):
        for key, store in (("k", small["k"]), ("v", small["v"])):
            t = np.full((1, D.heads, 32, D.head_dim), 0x7FC0, dtype=np.uint16)
            for p in range(50 - 32, 50):
                t[0, :, p % 32] = src[key][l][0, :, p % 64]
            store.append(t)
    Mbig = oracle.OracleModel(mnp)
    Mbig.dims = big
    ref, _ = oracle.oracle_round(Mbig, src)
    got, _ = oracle.oracle_round(M, small)
    assert np.all(np.isfinite(got))
    assert np.array_equal(got, ref)
    # poisoning the out-of-window rows of the big ring changes nothing
    pois = dict(src)
    pois["k"] = [t.copy() for t in src["k"]]
    pois["v"] = [t.copy() for t in src["v"]]
    for t in pois["k"] + pois["v"]:
        for p in range(0, 50 - 32):
            t[0, :, p % 64] = 0x7FC0
        t[0, :, 50:] = 0x7FC0
    got2, _ = oracle.oracle_round(Mbig, pois)
    assert np.array_equal(got2, ref)


def test_empty_context_attends_to_the_block_only(models):
    mnp, M = models["B"]
    cfg = dict(name="e", streams=2, lens=("const", 0), model="B", ingest=0)
    inp = synth.to_numpy_inputs(synth.make_inputs(cfg, D, vocab=torch.from_numpy(mnp["vocab"]),
                                                  poison=True))
    logits, ids = oracle.oracle_round(M, inp)
    assert np.all(np.isfinite(logits)) and np.all(ids >= 0)


def test_nan_logits_never_win():
    mnp = synth.to_numpy_model(synth.make_model(D, "A"))
    M = oracle.OracleModel(mnp)
    cfg = dict(name="n", streams=1, lens=("const", 4), model="A", ingest=0)
    inp = synth.to_numpy_inputs(synth.make_inputs(cfg, D, vocab=torch.from_numpy(mnp["vocab"])))
    base, ids = oracle.oracle_round(M, inp)
    M.head = M.head.copy()
    win = int(np.argmax(base[0, 0]))
    M.head[win] = np.nan
    got, ids2 = oracle.oracle_round(M, inp)
    row = np.where(np.isnan(got[0, 0]), -np.inf, got[0, 0])
    assert ids2[0, 0] == mnp["vocab"][int(np.argmax(row))] != ids[0, 0]
    M.head[:] = np.nan
    _, ids3 = oracle.oracle_round(M, inp)
    assert np.all(ids3 == -1)


def test_ingest_then_round_is_finite_and_moves_lengths(models):
    mnp, M = models["B"]
    cfg = dict(name="i", streams=2, lens=("const", 27), model="B", ingest=5)
    inp = synth.to_numpy_inputs(synth.make_inputs(cfg, D, vocab=torch.from_numpy(mnp["vocab"]),
                                                  poison=True))
    after = oracle.oracle_ingest(M, inp)
    assert np.array_equal(after["lens"], inp["lens"] + 5)
    # positions 27..31 land in slots 27..31; the ring then holds 32 valid rows
    for l in range(D.layers):
        assert not np.any(np.isnan(oracle.decode_bf16(after["k"][l])))
    logits, _ = oracle.oracle_round(M, after)
    assert np.all(np.isfinite(logits))


def test_depth_one_is_one_round_and_row0_ignores_depth(models, inputs):
    M = models["B"][1]
    one, ids1 = oracle.oracle_round(M, inputs)
    d1, i1 = oracle.oracle_round_depth(M, inputs, 1)
    assert np.array_equal(one, d1) and np.array_equal(ids1, i1)
    d2, _ = oracle.oracle_round_depth(M, inputs, 2)
    # row 0 never reads a predecessor (Position 1 bullet): identical at any depth
    assert np.array_equal(d2[:, 0], one[:, 0])
    assert not np.allclose(d2[:, 1:], one[:, 1:])


def test_depth_with_zero_predecessor_head_is_one_round(models, inputs):
    # model A's predecessor U is zero: predecessors cannot change any row
    M = models["A"][1]
    one, ids1 = oracle.oracle_round(M, inputs)
    d3, i3 = oracle.oracle_round_depth(M, inputs, 3)
    assert np.array_equal(one, d3) and np.array_equal(ids1, i3)


def test_bf16_head_is_the_full_head_gathered():
    # the card's Use section allows a bf16 head slice: the LM head's rows at
    # the draft vocabulary, unquantised
    m = synth.make_model(D, "C", head="bf16")
    mnp = synth.to_numpy_model(m)
    M = oracle.OracleModel(mnp)
    cfg = dict(name="h", streams=2, lens=("uniform", 1, 40), model="C", ingest=0)
    inp = synth.to_numpy_inputs(synth.make_inputs(cfg, D, vocab=m["vocab"]))
    logits, ids, x = oracle.oracle_round(M, inp, return_hidden=True)
    full = oracle.decode_bf16(mnp["table"])                           # [full_vocab][H]
    z = oracle.rmsnorm(x, M.final_norm, D.rms_eps)
    assert np.allclose((z @ full.T)[..., mnp["vocab"]], logits, rtol=1e-12, atol=1e-12)
    # the NVFP4 head of the same table drafts from nearby logits
    Mq = oracle.OracleModel({k: v for k, v in mnp.items() if k != "head_format"})
    lq, _ = oracle.oracle_round(Mq, inp)
    assert 0 < np.abs(lq - logits).max() < 0.2 * np.abs(logits).max()


def test_fp8_head_decodes_the_block_fp8_rows():
    m = synth.make_model(D, "B", head="fp8")
    mnp = synth.to_numpy_model(m)
    M = oracle.OracleModel(mnp)
    full = oracle.decode_bf16(mnp["table"])[mnp["vocab"]]
    # block-FP8 keeps each value within half an e4m3 step of the bf16 row:
    # 2^-4 relative for normals, half the subnormal step 2^-9 s below 2^-6 s
    # (s the block's scale), so the head is the bf16 head up to that rounding
    s = np.repeat(np.asarray(mnp["head_fp8.s"], dtype=np.float64), 64, axis=1)
    assert np.all(np.abs(M.head - full) <= np.abs(full) * 2.0 ** -4 + s * 2.0 ** -10 + 1e-15)
    assert not np.array_equal(M.head, full)


def test_body_formats_agree_where_all_three_are_exact():
    """The card's Use section allows FP8, NVFP4 and bf16 bodies. With weights
    every format holds exactly (an e2m1 value times a power-of-two scale per 16
    inputs times a power of two per matrix), the three decodes are the same
    matrices, so the rounds are identical in fp64. Block scales that vary
    every 16 inputs and tensor scales that vary by matrix make a wrong nibble
    order, scale repeat or dropped tensor scale show up."""
    base = synth.to_numpy_model(synth.make_model(D, "C"))
    rng = np.random.default_rng(5)
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    models = {f: dict(base, body_format=f) for f in ("fp8", "nvfp4", "bf16")}
    names = [k[:-2] for k in base if k.endswith(".q") and not k.startswith("head")]
    assert len(names) == 5 + 7 * D.layers + 2 * (D.layers - 1)
    e4m3 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    for name in names:
        rows, cols = base[name + ".q"].shape
        codes = rng.integers(0, 16, (rows, cols)).astype(np.uint8)
        val = np.where(codes >= 8, -1.0, 1.0) * mags[codes & 7]
        blk = np.exp2(rng.integers(-1, 3, (rows, cols // 16)).astype(np.float64))
        g = float(np.exp2(rng.integers(-9, -5)))
        w = val * np.repeat(blk, 16, axis=1) * g
        models["fp8"][name + ".q"] = e4m3(val * np.repeat(blk, 16, axis=1))
        models["fp8"][name + ".s"] = np.full((rows, cols // 64), g, dtype=np.float32)
        models["nvfp4"][name + ".q4"] = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
        models["nvfp4"][name + ".s4"] = e4m3(blk)
        models["nvfp4"][name + ".g"] = g
        models["bf16"][name + ".bf16"] = synth.bf16_bits(torch.from_numpy(w)).numpy().view(np.uint16)
    inp = synth.to_numpy_inputs(synth.make_inputs(CFG, D, vocab=torch.from_numpy(base["vocab"])))
    out = {f: oracle.oracle_round(oracle.OracleModel(m), inp) for f, m in models.items()}
    Ms = {f: oracle.OracleModel(m) for f, m in models.items()}
    assert np.array_equal(Ms["fp8"].fuse, Ms["nvfp4"].fuse) and np.array_equal(Ms["fp8"].fuse, Ms["bf16"].fuse)
    for f in ("nvfp4", "bf16"):
        assert np.array_equal(out[f][0], out["fp8"][0]), f
        assert np.array_equal(out[f][1], out["fp8"][1]), f
    # and the weights are not trivially shared: the decoded matrices differ from the model's own
    assert not np.array_equal(Ms["fp8"].fuse, oracle.OracleModel(base).fuse)
