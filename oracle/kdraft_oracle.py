"""Plain, slow fp64 oracle of one batched Kolibri-1 block-drafter round.

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``; never by the library.

Authority: the model card "Kolibri-1 block drafter", section "Architecture"
(bullets Input, Body, Position 1, Positions 2-4, Predecessor head, Spine,
Output, and the Serving paragraph for the weight formats). Where the card is
silent the plainest reading is taken and named in the function that uses it:

* rows 1-3 start as  mask + f + U_p silu(A_p f + B_p E[pred])  (an elementwise
  sum; only row 0 goes through the 5120->2560 projection);
* h in the predecessor head is the anchor's fused state f;
* row j (j = 1..3) uses pred[j-1], the token just before the one it drafts;
* the context-row input is [fused state ; embedding], in that order;
* the spine has one weight set per layer 2, 3, 4 and all rows read the
  layer input before any spine update;
* RMSNorm has eps = 1e-6 and a gain vector; no biases anywhere;
* RoPE is rotate-half over the whole head, frequencies theta^(-i/(d/2));
* block row j sits at position len + j; the context occupies [len - n, len)
  with n = min(len, window), stored at slot pos % capacity;
* every window row is visible to every block row; block row j sees block rows
  0..j; scores are scaled by 1/sqrt(head_dim);
* head rows are in draft-vocabulary order; ties go to the lowest draft index,
  NaN never wins, a row with no finite logit reports id -1;
* ingested K/V are rounded to bf16 (nearest even) because the cache is bf16;
  a rotated 4-bit cache follows the readings listed in kv_int4.

Every weight is decoded to its exact real value; activations are never
quantised. Integer data (ids, lengths) follow the same indexing as the card.
"""
from __future__ import annotations

import math

import numpy as np

from . import kv_int4


# ----------------------------------------------------------------------------
# Exact decoders (model card, "Architecture", Serving paragraph: block-FP8 is
# e4m3 with an fp32 scale per row and 64 inputs; the head slice is NVFP4).
# ----------------------------------------------------------------------------

def decode_e4m3(codes) -> np.ndarray:
    """OCP e4m3 (bias 7, no infinities, S.1111.111 is NaN) to float64."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & ((c & 7) == 7), np.nan, val)


def decode_e2m1(nibbles) -> np.ndarray:
    """OCP e2m1 (bias 1, one mantissa bit, no NaN/inf) to float64."""
    n = np.asarray(nibbles, dtype=np.int64) & 0xF
    sign = np.where((n >> 3) & 1, -1.0, 1.0)
    e = (n >> 1) & 3
    m = (n & 1).astype(np.float64)
    val = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0))
    return sign * val


def decode_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) to float64: the top half of an fp32."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """float64 -> nearest bf16 (ties to even), returned as uint16 bits."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.float64)
    fin = np.isfinite(x) & (x != 0)
    _, ex = np.frexp(np.where(fin, x, 1.0))
    lead = np.maximum(ex - 1, -126)                  # exponent of the leading bit
    q = np.exp2((lead - 7).astype(np.float64))       # bf16 keeps 8 significant bits
    r = np.rint(np.where(fin, x, 0.0) / q) * q       # np.rint rounds half to even
    out = np.where(fin, r, x)
    big = np.abs(out) > float(np.float32(3.3895313892515355e38))
    out = np.where(big & np.isfinite(out), np.copysign(np.inf, out), out)
    return (out.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def block_fp8(q, s) -> np.ndarray:
    """W[o][i] = e4m3(q[o][i]) * s[o][i // 64] (one scale per row per 64 inputs).
    The codes are decoded through the table of all 256 exact values."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.float64)
    return decode_e4m3(np.arange(256))[q] * np.repeat(s, 64, axis=1)


def nvfp4(q4, s4, g) -> np.ndarray:
    """W[o][i] = e2m1(code[o][i]) * e4m3(s4[o][i // 16]) * g; code of the even
    column in the low nibble of each byte."""
    q4 = np.asarray(q4, dtype=np.uint8)
    rows = q4.shape[0]
    codes = np.empty((rows, q4.shape[1] * 2), dtype=np.uint8)
    codes[:, 0::2] = q4 & 0xF
    codes[:, 1::2] = q4 >> 4
    scales = decode_e4m3(np.arange(256))[np.asarray(s4, dtype=np.uint8)]
    return decode_e2m1(np.arange(16))[codes] * np.repeat(scales, 16, axis=1) * float(np.float32(g))


# ----------------------------------------------------------------------------
# Elementwise pieces (model card, "Architecture": Body and Spine bullets)
# ----------------------------------------------------------------------------

def rmsnorm(x, g, eps) -> np.ndarray:
    """g * x / sqrt(mean(x^2) + eps) over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return np.asarray(g, dtype=np.float64) * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def silu(u) -> np.ndarray:
    u = np.asarray(u, dtype=np.float64)
    return u / (1.0 + np.exp(-u))


def rope(x, pos, theta) -> np.ndarray:
    """Rotary embedding, rotate-half form (model card, "Architecture", Body:
    RoPE theta 10,000). x [..., d]; pos broadcasts against x[..., 0]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    w = theta ** (-np.arange(half, dtype=np.float64) / half)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * w
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def attention(q, kc, vc, kb, vb) -> np.ndarray:
    """Block cross-attention for one stream (model card, "Architecture", Body:
    each layer cross-attends to the last 2,048 context rows; the block is causal
    inside itself).

    q, kb, vb: [rows][heads][d] block queries/keys/values; kc, vc: [heads][n][d]
    visible context keys/values. Row j sees every context row and block rows
    0..j. Softmax with the maximum subtracted; scores scaled by 1/sqrt(d).
    """
    rows, heads, d = q.shape
    scale = 1.0 / math.sqrt(d)
    sc = np.einsum("jhd,hnd->hjn", q, kc) * scale                # [h][rows][n]
    sb = np.einsum("jhd,ihd->hji", q, kb) * scale                # [h][rows][rows]
    causal = np.tril(np.ones((rows, rows), dtype=bool))
    sb = np.where(causal[None], sb, -np.inf)
    s = np.concatenate([sc, sb], axis=-1)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    n = kc.shape[1]
    o = np.einsum("hjn,hnd->jhd", p[..., :n], vc) + np.einsum("hji,ihd->jhd", p[..., n:], vb)
    return o


def top2_gap(logits) -> np.ndarray:
    """Top-1 minus top-2 logit per row (finite values only)."""
    z = np.where(np.isfinite(logits), logits, -np.inf)
    part = -np.sort(-z, axis=-1)[..., :2]
    return part[..., 0] - part[..., 1]


# ----------------------------------------------------------------------------
# Model: weights decoded once to fp64 (the analogue of a load step)
# ----------------------------------------------------------------------------

class OracleModel:
    """Decodes a synthetic model (numpy dict of codes/scales/bits) to fp64."""

    def __init__(self, m: dict, decode_table: bool = False):
        self.dims = d = m["dims"]
        # body matrices: block-FP8 (the card's serving format) or, as its Use
        # section allows, NVFP4 or bf16
        body = m.get("body_format", "fp8")
        if body == "nvfp4":
            W = lambda name: nvfp4(m[name + ".q4"], m[name + ".s4"], m[name + ".g"])
        elif body == "bf16":
            W = lambda name: decode_bf16(m[name + ".bf16"])
        else:
            W = lambda name: block_fp8(m[name + ".q"], m[name + ".s"])
        self.fuse = W("fuse")
        self.fc = W("fc")
        self.pred_a, self.pred_b, self.pred_u = W("pred_a"), W("pred_b"), W("pred_u")
        self.mask = np.asarray(m["mask"], dtype=np.float64)
        self.layers = []
        for l in range(d.layers):
            p = f"layers.{l}."
            L = dict(attn_norm=np.asarray(m[p + "attn_norm"], np.float64),
                     ffn_norm=np.asarray(m[p + "ffn_norm"], np.float64))
            for nm in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
                L[nm] = W(p + nm)
            if l >= 1:
                sp = f"spine.{l}."
                L["spine_norm"] = np.asarray(m[sp + "norm"], np.float64)
                L["spine_a"], L["spine_u"] = W(sp + "a"), W(sp + "u")
            self.layers.append(L)
        self.final_norm = np.asarray(m["final_norm"], np.float64)
        # the head slice: NVFP4 (the card's serving format) or, as its Use
        # section allows, bf16 or block-FP8
        if m.get("head_format") == "bf16":
            self.head = decode_bf16(m["head_bf16"])
        elif m.get("head_format") == "fp8":
            self.head = block_fp8(m["head_fp8.q"], m["head_fp8.s"])
        else:
            self.head = nvfp4(m["head.q4"], m["head.s4"], m["head.g"])
        self.vocab = np.asarray(m["vocab"], dtype=np.int64)
        self.table_bits = m["table"]           # bf16 bits; rows decoded on use
        # per-layer sign vectors of a rotated 4-bit cache (absent: bf16 only)
        rs = m.get("kv_rot_signs")
        self.kv_rot_signs = None if rs is None else np.asarray(rs, dtype=np.int64)

    def embed(self, ids) -> np.ndarray:
        return decode_bf16(self.table_bits[np.asarray(ids, dtype=np.int64)])


# ----------------------------------------------------------------------------
# The round
# ----------------------------------------------------------------------------

def _visible(length, dims):
    n = min(int(length), dims.window)
    pos = np.arange(int(length) - n, int(length))
    return pos, pos % dims.capacity


def _context_kv(M: OracleModel, inp: dict, l: int, b: int, slots):
    """The visible context keys and values of stream b, layer l, [heads][n][d].
    A bf16 cache holds them directly. A rotated 4-bit cache (the 4-bit KV
    cache article, section What we do) holds codes of R k and of v: the values are
    decoded, and the keys turned back by R^T, which leaves every score q.k
    as the rotated cache gives it, (R q).(R k)."""
    if inp.get("kv_format") == "int4":
        kr = kv_int4.decode_int4(inp["k"][l][b][:, slots, :], inp["k_so"][l][b][:, slots, :])
        vc = kv_int4.decode_int4(inp["v"][l][b][:, slots, :], inp["v_so"][l][b][:, slots, :])
        return kv_int4.unrotate_rows(kr, M.kv_rot_signs[l]), vc
    return decode_bf16(inp["k"][l][b][:, slots, :]), decode_bf16(inp["v"][l][b][:, slots, :])


def oracle_round(M: OracleModel, inp: dict, block: int | None = None,
                 spine: bool = True, return_hidden: bool = False, act=None):
    """One round for every stream; returns (logits [B][rows][VD], ids [B][rows]).

    Steps in the order of the model card's "Architecture" section:
      Input: f = W_fuse [t44; t47; t49]; row 0 = W_fc [f ; E[anchor]].
      Positions 2-4 / Predecessor head: row j = mask + f + U_p silu(A_p f + B_p E[pred[j-1]]).
      Body x4: (spine before layers 2-4) -> RMSNorm -> q,k,v -> RoPE -> attention
               -> W_o + residual -> RMSNorm -> SwiGLU FFN + residual.
      Output: RMSNorm -> head restricted to the draft vocabulary -> argmax.
    ``block`` < 4 runs a shorter block (block=1 is the chain-drafter row alone);
    ``spine=False`` zeroes the spine's contribution.
    ``act``: a function applied to every input of a weight product before it
    (a model of an activation number format, for precision studies); None
    keeps them exact.
    """
    q_ = (lambda t: t) if act is None else act
    d = M.dims
    R = d.block if block is None else block
    B = int(inp["streams"])
    H, NH, Dh = d.hidden, d.heads, d.head_dim
    taps = decode_bf16(inp["taps"]).reshape(B, d.taps * H)
    anchor = np.asarray(inp["anchor"]).reshape(B)
    pred = np.asarray(inp["pred"]).reshape(B, d.block - 1)
    lens = np.asarray(inp["lens"]).reshape(B)

    # Input: tap fuse, then the anchor row in the EAGLE-3 context-row form.
    f = q_(taps) @ M.fuse.T                                           # [B][H]
    x = np.zeros((B, R, H))
    x[:, 0] = q_(np.concatenate([f, M.embed(anchor)], axis=1)) @ M.fc.T
    # Positions 2-4: mask row + anchor's fused state + predecessor term.
    for j in range(1, R):
        u = q_(f) @ M.pred_a.T + q_(M.embed(pred[:, j - 1])) @ M.pred_b.T
        x[:, j] = M.mask + f + q_(silu(u)) @ M.pred_u.T

    pos_blk = lens[:, None] + np.arange(R)[None, :]                   # [B][R]
    for l, L in enumerate(M.layers):
        if l >= 1 and spine:
            # Spine: row j reads row j-1 of the layer input (simultaneous update).
            src = x[:, : R - 1]
            add = q_(silu(q_(rmsnorm(src, L["spine_norm"], d.rms_eps)) @ L["spine_a"].T)) @ L["spine_u"].T
            x = x.copy()
            x[:, 1:] += add
        a = q_(rmsnorm(x, L["attn_norm"], d.rms_eps))
        q = (a @ L["wq"].T).reshape(B, R, NH, Dh)
        k = (a @ L["wk"].T).reshape(B, R, NH, Dh)
        v = (a @ L["wv"].T).reshape(B, R, NH, Dh)
        q = rope(q, pos_blk[:, :, None], d.rope_theta)
        k = rope(k, pos_blk[:, :, None], d.rope_theta)
        o = np.empty((B, R, NH, Dh))
        for b in range(B):
            _, slots = _visible(lens[b], d)
            kc, vc = _context_kv(M, inp, l, b, slots)
            o[b] = attention(q[b], kc, vc, k[b], v[b])
        x = x + q_(o.reshape(B, R, H)) @ L["wo"].T
        c = q_(rmsnorm(x, L["ffn_norm"], d.rms_eps))
        x = x + q_(silu(c @ L["w_gate"].T) * (c @ L["w_up"].T)) @ L["w_down"].T

    z = rmsnorm(x, M.final_norm, d.rms_eps)
    logits = q_(z) @ M.head.T                                         # [B][R][VD]
    masked = np.where(np.isfinite(logits), logits, -np.inf)
    best = np.argmax(masked, axis=-1)                                 # first maximum
    ok = np.isfinite(masked.max(axis=-1))
    ids = np.where(ok, M.vocab[best], -1)
    if return_hidden:
        return logits, ids, x
    return logits, ids


def oracle_round_depth(M: OracleModel, inp: dict, depth: int):
    """`depth` rounds in a row (model card, "Architecture", Serving: several
    drafter rounds run before the target verifies; Predecessor head: at serving
    the token before a row is the drafter's own previous draft). Round 1 takes
    the given predecessor ids; round r+1 takes pred[b][j-1] = round r's draft
    of block row j-1. Returns the last round's (logits, ids)."""
    cur = dict(inp)
    for r in range(depth):
        logits, ids = oracle_round(M, cur)
        cur = dict(cur, pred=np.asarray(ids)[:, : M.dims.block - 1].copy())
    return logits, ids


def oracle_ingest(M: OracleModel, inp: dict, return_exact: bool = False):
    """Append new context rows (model card, "Architecture", Input: context rows
    are [fused state ; embedding of the next token] -> 5120->2560; Body: the
    cached K/V each layer attends to).

    Every layer projects the same row c through its attention RMSNorm and
    W_k / W_v; K gets RoPE at its absolute position; both are rounded to bf16
    and stored at slot pos % capacity; len grows by the number of rows.
    With a rotated 4-bit cache (kv_format "int4"; the 4-bit KV cache
    article, section What we do) K is rotated by the layer's R after RoPE, and both K and V
    are stored as codes with their fp16 scale and offset instead.
    Returns a new input dict (K/V copies and lengths updated); with
    return_exact also the unrounded fp64 K (rotated, for a 4-bit cache) and V
    per layer ([B][n][heads][d]).
    """
    d = M.dims
    B = int(inp["streams"])
    H, NH, Dh = d.hidden, d.heads, d.head_dim
    taps = decode_bf16(inp["ingest_taps"])                            # [B][n][3][H]
    n_new = taps.shape[1]
    nxt = np.asarray(inp["ingest_ids"]).reshape(B, n_new)
    lens = np.asarray(inp["lens"]).reshape(B).astype(np.int64)
    out = dict(inp)
    int4 = inp.get("kv_format") == "int4"
    out["k"] = [k.copy() for k in inp["k"]]
    out["v"] = [v.copy() for v in inp["v"]]
    if int4:
        out["k_so"] = [t.copy() for t in inp["k_so"]]
        out["v_so"] = [t.copy() for t in inp["v_so"]]
    f = taps.reshape(B, n_new, d.taps * H) @ M.fuse.T
    c = np.concatenate([f, M.embed(nxt)], axis=-1) @ M.fc.T           # [B][n][H]
    pos = lens[:, None] + np.arange(n_new)[None, :]
    exact = []
    for l, L in enumerate(M.layers):
        a = rmsnorm(c, L["attn_norm"], d.rms_eps)
        k = rope((a @ L["wk"].T).reshape(B, n_new, NH, Dh), pos[:, :, None], d.rope_theta)
        v = (a @ L["wv"].T).reshape(B, n_new, NH, Dh)
        if int4:
            k = kv_int4.rotate_rows(k, M.kv_rot_signs[l])
            (kq, kso), (vq, vso) = kv_int4.quantize_int4(k), kv_int4.quantize_int4(v)
        else:
            kb, vb = round_bf16(k), round_bf16(v)
        exact.append((k, v))
        for b in range(B):
            for i in range(n_new):
                slot = int(pos[b, i]) % d.capacity
                if int4:
                    out["k"][l][b][:, slot, :] = kq[b, i]
                    out["v"][l][b][:, slot, :] = vq[b, i]
                    out["k_so"][l][b][:, slot, :] = kso[b, i]
                    out["v_so"][l][b][:, slot, :] = vso[b, i]
                else:
                    out["k"][l][b][:, slot, :] = kb[b, i]
                    out["v"][l][b][:, slot, :] = vb[b, i]
    out["lens"] = (lens + n_new).astype(np.int32)
    return (out, exact) if return_exact else out
