"""Pins of the rotated 4-bit K/V cache in the oracle.

The article "Serving Kolibri-1 with a 4-bit KV cache" (section What we do)
fixes R = H diag(s) / sqrt(d) with H the Hadamard matrix,
keys rotated before caching and queries by the same R (q.k unchanged), and
4-bit codes with one fp16 scale and offset per token and head; values are not
rotated. The pins below tie each step to something outside the oracle: the
textbook Sylvester matrix and scipy's construction, hand-worked bytes, the
quantiser's half-step error bound, and round-level equivalences with a bf16
cache that holds exactly the same keys and values.
"""
import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
import synth
from oracle import kv_int4

D = synth.TINY


def test_hadamard_matches_textbook_and_scipy():
    h4 = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]], dtype=float)
    assert np.array_equal(kv_int4.hadamard(4), h4)
    for n in (1, 2, 8, 64, 128):
        h = kv_int4.hadamard(n)
        assert np.array_equal(h, scipy.linalg.hadamard(n).astype(float))
        assert np.array_equal(h @ h.T, n * np.eye(n))


def test_rotation_is_orthogonal_and_keeps_dot_products():
    rng = np.random.default_rng(5)
    for d in (64, 128):
        s = rng.choice([-1, 1], size=d)
        R = kv_int4.rotation(s)
        assert np.allclose(R @ R.T, np.eye(d), atol=1e-14)
        # R = H diag(s)/sqrt(d): column j is s_j times column j of H over sqrt(d)
        H = scipy.linalg.hadamard(d).astype(float)
        assert np.allclose(R, H * s[None, :] / np.sqrt(d), atol=0)
        q, k = rng.standard_normal((2, 5, d))
        qr, kr = kv_int4.rotate_rows(q, s), kv_int4.rotate_rows(k, s)
        assert np.allclose(np.sum(qr * kr, -1), np.sum(q * k, -1), rtol=1e-13)
        assert np.allclose(kv_int4.unrotate_rows(kr, s), k, atol=1e-13)


def test_decode_hand_worked_bytes():
    # byte 0x21: dim 0 (low nibble) code 1, dim 1 code 2; byte 0xF0: 0 and 15
    packed = np.array([[0x21, 0xF0]], dtype=np.uint8)
    so = np.array([[np.float16(0.5).view(np.uint16), np.float16(-1.0).view(np.uint16)]])
    got = kv_int4.decode_int4(packed, so)
    assert np.array_equal(got, [[-0.5, 0.0, -1.0, 6.5]])
    assert np.array_equal(kv_int4.pack_codes(kv_int4.unpack_codes(packed)), packed)


def test_quantize_worked_examples():
    # an evenly spaced row: range 7.5 over 15 steps, every value on a code
    x = -3.0 + 0.5 * np.arange(16)
    q, so = kv_int4.quantize_int4(x)
    assert np.array_equal(kv_int4.unpack_codes(q), np.arange(16))
    assert kv_int4.decode_f16(so).tolist() == [0.5, -3.0]
    assert np.array_equal(kv_int4.decode_int4(q, so), x)
    # ties go to the even code: (x - 0)/1 = 2.5 -> 2, 3.5 -> 4
    x = np.array([0.0, 15.0, 2.5, 3.5])
    q, so = kv_int4.quantize_int4(x)
    assert kv_int4.unpack_codes(q).tolist() == [0, 15, 2, 4]
    # a constant row: zero scale, every code 0, the value is fp16(offset)
    x = np.full(8, 0.1)
    q, so = kv_int4.quantize_int4(x)
    assert kv_int4.decode_f16(so)[0] == 0.0
    assert np.all(kv_int4.unpack_codes(q) == 0)
    assert np.all(kv_int4.decode_int4(q, so) == float(np.float16(0.1)))


def test_round_f16_is_nearest_even():
    # 1 + 2^-11 is halfway between 1 and 1 + 2^-10: ties to the even mantissa (1)
    assert kv_int4.decode_f16(kv_int4.round_f16(1 + 2.0 ** -11)) == 1.0
    assert kv_int4.decode_f16(kv_int4.round_f16(1 + 3 * 2.0 ** -11)) == 1 + 2.0 ** -9
    assert kv_int4.decode_f16(kv_int4.round_f16(1 + 2.0 ** -11 + 2.0 ** -30)) == 1 + 2.0 ** -10


def test_quantize_error_is_half_a_step():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((200, 128)) * rng.uniform(0.01, 10, (200, 1))
    q, so = kv_int4.quantize_int4(x)
    y = kv_int4.decode_int4(q, so)
    sc, off = (kv_int4.decode_f16(so)[..., i] for i in (0, 1))
    top = off + 15 * sc
    inside = (x >= off[:, None]) & (x <= top[:, None])
    err = np.abs(y - x)
    assert np.all(err[inside] <= (sc[:, None] / 2 * (1 + 1e-12) + 0 * x)[inside])
    # outside [offset, offset + 15 scale] only by fp16 rounding of min and scale
    slack = np.maximum(off - x.min(-1), 0) + np.maximum(x.max(-1) - top, 0)
    assert np.all(err <= sc[:, None] / 2 + slack[:, None] + 1e-12)
    assert np.all(slack <= 2.0 ** -10 * (np.abs(x).max(-1)) * 8)


@pytest.fixture(scope="module")
def model_b():
    m = synth.to_numpy_model(synth.make_model(D, "B"))
    return m, oracle.OracleModel(m)


def test_synthetic_signs_are_plus_minus_one(model_b):
    m, _ = model_b
    s = m["kv_rot_signs"]
    assert s.shape == (D.layers, D.head_dim)
    assert set(np.unique(s)) == {-1, 1}


def _one_hot_int4_and_bf16(m, lens):
    """A 4-bit cache whose rotated keys are t * e_dim (code 1 at one dimension,
    scale t, offset 0) and whose values are -1 + code/8, next to the bf16 cache
    holding the same keys unrotated, R^T (t e_dim) = t s * H[dim, :] / sqrt(d)
    (built with scipy's Hadamard matrix), and the same values. Every number is
    exact in bf16."""
    rng = np.random.default_rng(11)
    B, NH, C, d = len(lens), D.heads, D.capacity, D.head_dim
    H = scipy.linalg.hadamard(d).astype(float)
    int4 = {"kv_format": "int4", "k": [], "v": [], "k_so": [], "v_so": []}
    bf = {"k": [], "v": []}
    f16 = lambda v: np.float16(v).view(np.uint16)
    for l in range(D.layers):
        s = m["kv_rot_signs"][l].astype(float)
        dim = rng.integers(0, d, (B, NH, C))
        t = rng.choice([0.5, 1.0, 1.5, -2.0], (B, NH, C))
        codes = np.zeros((B, NH, C, d), dtype=np.int64)
        np.put_along_axis(codes, dim[..., None], 1, axis=-1)
        kso = np.zeros((B, NH, C, 2), dtype=np.uint16)
        kso[..., 0] = np.vectorize(f16)(t)
        kso[..., 1] = f16(0.0)
        key = t[..., None] * s[None, None, None, :] * H[dim] / np.sqrt(d)
        vcodes = rng.integers(0, 16, (B, NH, C, d))
        vso = np.zeros((B, NH, C, 2), dtype=np.uint16)
        vso[..., 0], vso[..., 1] = f16(0.125), f16(-1.0)
        val = -1.0 + vcodes / 8.0
        int4["k"].append(kv_int4.pack_codes(codes))
        int4["v"].append(kv_int4.pack_codes(vcodes))
        int4["k_so"].append(kso)
        int4["v_so"].append(vso)
        kb, vb = oracle.round_bf16(key), oracle.round_bf16(val)
        assert np.array_equal(oracle.decode_bf16(kb), key)
        assert np.array_equal(oracle.decode_bf16(vb), val)
        bf["k"].append(kb)
        bf["v"].append(vb)
    return int4, bf


def test_round_on_rotated_cache_equals_round_on_the_plain_keys(model_b):
    m, M = model_b
    cfg = dict(name="r", streams=3, lens=("uniform", 1, 60), model="B", ingest=0)
    base = synth.to_numpy_inputs(synth.make_inputs(cfg, D, vocab=torch.from_numpy(m["vocab"])))
    int4, bf = _one_hot_int4_and_bf16(m, base["lens"])
    ref, ids_ref = oracle.oracle_round(M, dict(base, **bf))
    got, ids = oracle.oracle_round(M, dict(base, **int4))
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(ids, ids_ref)
    # the transposed rotation (R instead of R^T) would give other keys
    wrong = dict(base, **bf)
    wrong["k"] = []
    H = scipy.linalg.hadamard(D.head_dim).astype(float)
    for l in range(D.layers):
        s = m["kv_rot_signs"][l].astype(float)
        kr = kv_int4.decode_int4(int4["k"][l], int4["k_so"][l])
        wrong["k"].append(oracle.round_bf16(kr @ (H * s[None, :]).T / np.sqrt(D.head_dim)))
    bad, _ = oracle.oracle_round(M, wrong)
    assert not np.allclose(bad, ref, rtol=1e-6, atol=1e-6)


def test_synthetic_int4_cache_layout_and_poison(model_b):
    m, M = model_b
    cfg = dict(name="q", streams=2, lens=("const", 20), model="B", ingest=0)
    inp = synth.to_numpy_inputs(synth.make_inputs(cfg, D, vocab=torch.from_numpy(m["vocab"]),
                                                  poison=True, kv="int4"))
    assert inp["k"][0].shape == (2, D.heads, D.capacity, D.head_dim // 2)
    assert inp["k_so"][0].shape == (2, D.heads, D.capacity, 2)
    so = kv_int4.decode_f16(inp["k_so"][0])
    assert np.all(np.isnan(so[:, :, 20:])) and np.all(np.isfinite(so[:, :, :20]))
    logits, ids = oracle.oracle_round(M, inp)
    assert np.all(np.isfinite(logits)) and np.all(ids >= 0)


def test_int4_ingest_stores_quantised_rotated_keys(model_b):
    m, M = model_b
    cfg = dict(name="iq", streams=2, lens=("const", 27), model="B", ingest=5)
    bf = synth.to_numpy_inputs(synth.make_inputs(cfg, D, vocab=torch.from_numpy(m["vocab"]),
                                                 poison=True))
    q4 = synth.to_numpy_inputs(synth.make_inputs(cfg, D, vocab=torch.from_numpy(m["vocab"]),
                                                 poison=True, kv="int4"))
    q4["ingest_taps"], q4["ingest_ids"] = bf["ingest_taps"], bf["ingest_ids"]
    _, exact_bf = oracle.oracle_ingest(M, bf, return_exact=True)
    after, exact_q = oracle.oracle_ingest(M, q4, return_exact=True)
    assert np.array_equal(after["lens"], q4["lens"] + 5)
    H = scipy.linalg.hadamard(D.head_dim).astype(float)
    for l in range(D.layers):
        s = m["kv_rot_signs"][l].astype(float)
        k_plain, v_plain = exact_bf[l]
        k_rot = k_plain @ (H * s[None, :]).T / np.sqrt(D.head_dim)
        assert np.allclose(exact_q[l][0], k_rot, atol=1e-12)
        for b in range(2):
            for i in range(5):
                slot = 27 + i
                for key, ref in (("k", k_rot), ("v", v_plain)):
                    y = kv_int4.decode_int4(after[key][l][b][:, slot], after[key + "_so"][l][b][:, slot])
                    x = ref[b, i]                                  # [heads][d]
                    sc = kv_int4.decode_f16(after[key + "_so"][l][b][:, slot, 0])
                    assert np.all(np.abs(y - x) <= sc[:, None] / 2 + 2.0 ** -10 * np.abs(x).max())
        # untouched slots keep their codes
        assert np.array_equal(after["k"][l][:, :, :27], q4["k"][l][:, :, :27])
    logits, _ = oracle.oracle_round(M, after)
    assert np.all(np.isfinite(logits))
