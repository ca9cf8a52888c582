"""Pins of the oracle's decoders and of the generator's quantisers.

Decoders are checked exhaustively against library casts (torch's
float8_e4m3fn and bfloat16) and against the OCP e2m1 value list; the matrix
decoders are checked against the quantisation error bound of the weights they
came from, which fails for a wrong scale index or a transposed layout.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.isnan(ours).sum() == 2          # S.1111.111
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_bf16_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])


def test_round_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000) * 10.0 ** rng.integers(-40, 38, 200000),
                        [0.0, -0.0, 1e-40, -3e-39, 3.4e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = oracle.round_bf16(x32.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_round_bf16_is_nearest_even_on_fp64_inputs():
    # Brute force: the two bf16 neighbours of x, the nearer wins, ties to the
    # even code. Inputs are fp64 values that fp32 cannot hold.
    rng = np.random.default_rng(2)
    x = rng.standard_normal(5000) * 3.0
    x += 2.0 ** -40
    ours = oracle.round_bf16(x)
    for xi, oi in zip(x, ours):
        lo = np.uint16(np.float32(xi).view(np.uint32) >> 16)     # truncation toward 0
        cands = [int(lo), int(lo) + 1]
        vals = [oracle.decode_bf16(np.uint16(c)) for c in cands]
        dist = [abs(float(v) - xi) for v in vals]
        if dist[0] < dist[1]:
            want = cands[0]
        elif dist[1] < dist[0]:
            want = cands[1]
        else:
            want = cands[0] if cands[0] % 2 == 0 else cands[1]
        assert int(oi) == want


def test_e2m1_matches_ocp_value_list():
    table = np.loadtxt(os.path.join(GOLDEN, "e2m1_values.txt"))
    codes = table[:, 0].astype(np.int64)
    vals = table[:, 1]
    assert np.array_equal(oracle.decode_e2m1(codes), vals)
    assert np.array_equal(oracle.decode_e2m1(codes + 8), -vals)


def test_e2m1_through_torch_e4m3():
    # e2m1 (bias 1, 1 mantissa bit) embeds in e4m3 (bias 7, 3 mantissa bits):
    # exponent field + 6, mantissa bit moved to the top mantissa position;
    # the subnormal 0.5 is the e4m3 normal with exponent field 6.
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        if e == 0:
            e8 = (s << 7) | ((6 << 3) if m else 0)
        else:
            e8 = (s << 7) | ((e + 6) << 3) | (m << 2)
        ref = torch.tensor([e8], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item()
        assert oracle.decode_e2m1(np.array([c]))[0] == ref


def test_e2m1_quantiser_roundtrip():
    codes = np.arange(16)
    vals = torch.from_numpy(oracle.decode_e2m1(codes)).float()
    back = synth.e2m1_codes(vals).numpy()
    want = codes.copy()
    want[8] = 0                                  # -0 is written as +0
    assert np.array_equal(back, want)


def _fp8_bound_ok(w, W, s):
    rows, cols = w.shape
    sb = np.repeat(s.astype(np.float64), 64, axis=1)
    y = np.abs(w / sb)
    bound = sb * np.maximum(y * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6)
    return np.all(np.abs(W - w) <= bound + 1e-30)


def test_block_fp8_decode_within_quantisation_bound():
    g = torch.Generator().manual_seed(3)
    # rows with very different magnitudes, so a wrong scale index is caught
    w = torch.randn(96, 320, generator=g) * torch.logspace(-3, 1, 96)[:, None]
    w[:, 64:128] *= 50.0
    q, s = synth.quant_block_fp8(w)
    W = oracle.block_fp8(q.numpy(), s.numpy())
    assert _fp8_bound_ok(w.double().numpy(), W, s.numpy())
    # the same codes read with the block scales in the wrong order must not pass
    s_wrong = np.ascontiguousarray(s.numpy()[:, ::-1])
    assert not _fp8_bound_ok(w.double().numpy(), oracle.block_fp8(q.numpy(), s_wrong), s.numpy())


def test_nvfp4_decode_within_quantisation_bound():
    g = torch.Generator().manual_seed(4)
    w = torch.randn(40, 256, generator=g) * 0.02
    w[:, 16:32] *= 30.0
    q4, s4, gs = synth.quant_nvfp4(w)
    W = oracle.nvfp4(q4.numpy(), s4.numpy(), gs)
    sb = np.repeat(oracle.decode_e4m3(s4.numpy()), 16, axis=1) * gs
    err = np.abs(W - w.double().numpy())
    assert np.all(err <= sb * 1.0 * (1 + 1e-6) + 1e-30)     # half spacing <= 1 at the top
    y = np.abs(w.double().numpy()) / np.where(sb > 0, sb, 1)
    small = y <= 1.75
    assert np.all(err[small] <= sb[small] * 0.25 * (1 + 1e-6) + 1e-30)
    assert float(np.abs(W).max()) > 0


def test_nvfp4_restricted_head_equals_gathered_full_head():
    g = torch.Generator().manual_seed(5)
    table = (torch.randn(500, 128, generator=g) * 0.02).to(torch.bfloat16).float()
    vocab = torch.sort(torch.randperm(500, generator=g)[:77]).values
    q4s, s4s, gslice = synth.quant_nvfp4(table[vocab])
    q4f, s4f, _ = synth.quant_nvfp4(table, g=gslice)
    restricted = oracle.nvfp4(q4s.numpy(), s4s.numpy(), gslice)
    full = oracle.nvfp4(q4f.numpy(), s4f.numpy(), gslice)
    assert np.array_equal(restricted, full[vocab.numpy()])
