"""Pins of the oracle's elementwise pieces and of its block attention.

RMSNorm: closed forms. RoPE: identity at position 0, a worked rotation, norm
preservation, the complex-number form and relative-position invariance.
Attention: an explicit loop over keys, torch's fp64 scaled_dot_product_attention
with a boolean mask, and closed forms (equal keys give the mean of the visible
values; a single dominant key gives its value).
"""
import math

import numpy as np
import torch

import oracle


def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64)) * 3.0
    y = oracle.rmsnorm(x, np.ones(64), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-13)
    assert np.allclose(oracle.rmsnorm(7.5 * x, np.ones(64), 0.0), y, rtol=1e-13)
    g = rng.standard_normal(64)
    assert np.allclose(oracle.rmsnorm(x, g, 0.0), g * y, rtol=1e-13)
    # eps enters under the root: a constant vector c*1 maps to c/sqrt(c^2+eps)
    c = np.full((1, 64), 0.01)
    assert np.allclose(oracle.rmsnorm(c, np.ones(64), 1e-4), 0.01 / math.sqrt(1e-4 + 1e-4))


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert np.isclose(oracle.silu(1.0), 1.0 / (1.0 + math.exp(-1.0)))
    assert np.isclose(oracle.silu(-50.0), -50.0 * math.exp(-50.0), rtol=1e-10)


def test_rope_position_zero_and_first_pair():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(128)
    assert np.array_equal(oracle.rope(x, 0, 1e4), x)
    # frequency 0 is 1 rad per position: e_0 rotates into e_64 as (cos p, sin p)
    e0 = np.zeros(128)
    e0[0] = 1.0
    y = oracle.rope(e0, 2.0, 1e4)
    assert np.isclose(y[0], math.cos(2.0)) and np.isclose(y[64], math.sin(2.0))
    assert np.allclose(np.delete(y, [0, 64]), 0.0)
    # the last frequency is theta^(-63/64)
    e63 = np.zeros(128)
    e63[63] = 1.0
    p = 1000.0
    w = 1e4 ** (-63 / 64)
    y = oracle.rope(e63, p, 1e4)
    assert np.isclose(y[63], math.cos(p * w)) and np.isclose(y[127], math.sin(p * w))


def test_rope_complex_form_norm_and_relative_invariance():
    rng = np.random.default_rng(2)
    d = 128
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for p in (0, 1, 17, 2047, 4099):
        z = q[:64] + 1j * q[64:]
        w = 1e4 ** (-np.arange(64) / 64)
        zr = z * np.exp(1j * p * w)
        y = oracle.rope(q, p, 1e4)
        assert np.allclose(y[:64], zr.real, atol=1e-12) and np.allclose(y[64:], zr.imag, atol=1e-12)
        assert np.isclose(np.linalg.norm(y), np.linalg.norm(q))
    a = oracle.rope(q, 2051, 1e4) @ oracle.rope(k, 37, 1e4)
    b = oracle.rope(q, 2051 - 37, 1e4) @ oracle.rope(k, 0, 1e4)
    assert np.isclose(a, b, rtol=1e-9)


def _loop_attention(q, kc, vc, kb, vb):
    rows, heads, d = q.shape
    n = kc.shape[1]
    out = np.zeros_like(q)
    for j in range(rows):
        for h in range(heads):
            keys = [kc[h, i] for i in range(n)] + [kb[i, h] for i in range(j + 1)]
            vals = [vc[h, i] for i in range(n)] + [vb[i, h] for i in range(j + 1)]
            scores = [sum(q[j, h, t] * key[t] for t in range(d)) / math.sqrt(d) for key in keys]
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            tot = sum(w)
            for t in range(d):
                out[j, h, t] = sum(wi * v[t] for wi, v in zip(w, vals)) / tot
    return out


def _rand_attn(rng, rows=4, heads=2, d=8, n=6):
    return (rng.standard_normal((rows, heads, d)), rng.standard_normal((heads, n, d)),
            rng.standard_normal((heads, n, d)), rng.standard_normal((rows, heads, d)),
            rng.standard_normal((rows, heads, d)))


def test_attention_matches_explicit_loops():
    rng = np.random.default_rng(3)
    for n in (0, 1, 6):
        args = _rand_attn(rng, n=n)
        assert np.allclose(oracle.attention(*args), _loop_attention(*args), rtol=1e-12, atol=1e-12)


def test_attention_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(4)
    rows, heads, d, n = 4, 3, 16, 37
    q, kc, vc, kb, vb = _rand_attn(rng, rows, heads, d, n)
    K = np.concatenate([kc, kb.transpose(1, 0, 2)], axis=1)          # [h][n+rows][d]
    V = np.concatenate([vc, vb.transpose(1, 0, 2)], axis=1)
    mask = np.ones((rows, n + rows), dtype=bool)
    mask[:, n:] = np.tril(np.ones((rows, rows), dtype=bool))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.transpose(1, 0, 2)), torch.from_numpy(K), torch.from_numpy(V),
        attn_mask=torch.from_numpy(mask)).numpy().transpose(1, 0, 2)
    assert np.allclose(oracle.attention(q, kc, vc, kb, vb), ref, rtol=1e-12, atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(5)
    rows, heads, d, n = 4, 2, 8, 5
    q, _, vc, _, vb = _rand_attn(rng, rows, heads, d, n)
    key = rng.standard_normal(d)
    kc = np.broadcast_to(key, (heads, n, d)).copy()
    kb = np.broadcast_to(key, (rows, heads, d)).copy()
    o = oracle.attention(q, kc, vc, kb, vb)
    for j in range(rows):
        want = (vc.sum(axis=1) + vb[: j + 1].sum(axis=0)) / (n + j + 1)
        assert np.allclose(o[j], want, rtol=1e-12)
    # one context key aligned with a huge query dominates every row
    kc2 = rng.standard_normal((heads, n, d)) * 0.01
    kc2[:, 2] = 1.0
    q2 = np.full((rows, heads, d), 400.0)
    kb2 = rng.standard_normal((rows, heads, d)) * 0.01
    o2 = oracle.attention(q2, kc2, vc, kb2, vb)
    assert np.allclose(o2, np.broadcast_to(vc[:, 2], (rows, heads, d)), atol=1e-9)


def test_top2_gap_hand_worked_rows():
    """The gap that decides which rows the id rule gates (the card's Output
    bullet: the draft is the argmax of the restricted logits). Hand-worked
    rows: the top two of each row by hand, non-finite logits ignored."""
    rows = np.array([
        [1.0, 3.0, 2.5, -7.0],                     # top 3.0, second 2.5
        [2.0, 2.0, 1.0, 0.0],                      # exact tie at the top
        [np.nan, 1.0, 0.25, 0.5],                  # NaN never counts
        [-np.inf, 5.0, -np.inf, -np.inf],          # one finite logit: nothing competes
        [-3.0, -1.0, -2.0, -1.5],                  # all negative: -1 vs -1.5
        [np.inf, 1.0, 0.0, -1.0],                  # +inf is not a finite logit
        [0.0, -0.5, 0.0625, 0.0],                  # the top one is not first
    ])
    want = np.array([0.5, 0.0, 0.5, np.inf, 0.5, 1.0, 0.0625])
    got = oracle.top2_gap(rows)
    assert got.shape == (7,)
    assert np.array_equal(got, want)
    # no finite logit at all: no gap (NaN), so such a row is never gated
    assert np.isnan(oracle.top2_gap(np.array([[np.nan, -np.inf, np.inf]])))[0]
    # works on the last axis of any batch shape
    batch = rows.reshape(7, 1, 4).repeat(3, axis=1)
    assert np.array_equal(oracle.top2_gap(batch), np.repeat(want[:, None], 3, axis=1))
    # the gate the GPU tests apply: gap > 1e-2
    assert (oracle.top2_gap(rows) > 1e-2).tolist() == [True, False, True, True, True, True, True]
