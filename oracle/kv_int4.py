"""Rotated 4-bit K/V cache: plain fp64 definitions.

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``; never by the library.

Authority: the article "Serving Kolibri-1 with a 4-bit KV cache", section
What we do. Per attention layer a fixed matrix R = H diag(s) / sqrt(d)
(H the d x d Hadamard matrix, s one random sign per column) rotates every key
before it is cached and every query the same way, so q.k is unchanged
(R is orthogonal). Keys and values are stored as 4-bit codes with one fp16
scale and one fp16 offset per token and head; values are not rotated.

Readings where the article is silent (each listed with the other readings):
* H is the Sylvester Hadamard matrix, H[i][j] = (-1)^popcount(i & j);
* the codes are asymmetric (min/max) uniform codes: scale = fp16((max -
  min) / 15), offset = fp16(min), code = clamp(round_half_even((x - offset) /
  scale), 0, 15), value = scale * code + offset; a zero scale gives code 0;
* the rotated key is the key after RoPE (the cache holds what the scores
  read); the drafter has no QK-norm gains, so nothing is folded into the query;
* two codes per byte, the even dimension in the low nibble.
"""
from __future__ import annotations

import math

import numpy as np


def hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two), from its entry
    formula (-1)^popcount(i & j)."""
    assert n > 0 and n & (n - 1) == 0
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    x = i & j
    pop = np.zeros_like(x)
    while np.any(x):
        pop += x & 1
        x >>= 1
    return np.where(pop % 2 == 0, 1.0, -1.0)


def rotation(signs) -> np.ndarray:
    """R = H diag(s) / sqrt(d) for one layer's sign vector s (entries +-1)."""
    s = np.asarray(signs, dtype=np.float64)
    d = s.shape[0]
    return hadamard(d) * s[None, :] / math.sqrt(d)


def decode_f16(bits) -> np.ndarray:
    """fp16 bit patterns -> exact fp64 values."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def round_f16(x) -> np.ndarray:
    """fp64 -> fp16 bits, round to nearest even (numpy's double-to-half cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def unpack_codes(packed) -> np.ndarray:
    """[..., d/2] bytes -> [..., d] codes 0..15 (even dimension = low nibble)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int64)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def pack_codes(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def decode_int4(packed, so_bits) -> np.ndarray:
    """Stored 4-bit rows -> their values: scale * code + offset per row.
    packed [..., d/2] uint8, so_bits [..., 2] uint16 (scale, offset)."""
    so = decode_f16(so_bits)
    return so[..., 0:1] * unpack_codes(packed) + so[..., 1:2]


def quantize_int4(x):
    """Rows x [..., d] (fp64) -> (packed codes [..., d/2], so bits [..., 2])."""
    x = np.asarray(x, dtype=np.float64)
    lo = x.min(axis=-1)
    hi = x.max(axis=-1)
    sb = round_f16((hi - lo) / 15.0)
    ob = round_f16(lo)
    scale = decode_f16(sb)[..., None]
    off = decode_f16(ob)[..., None]
    safe = np.where(scale > 0, scale, 1.0)
    code = np.where(scale > 0, np.clip(np.rint((x - off) / safe), 0, 15), 0)
    return pack_codes(code.astype(np.int64)), np.stack([sb, ob], axis=-1)


def rotate_rows(x, signs) -> np.ndarray:
    """R x for every row x [..., d] (as row vectors: x @ R^T)."""
    return np.asarray(x, dtype=np.float64) @ rotation(signs).T


def unrotate_rows(y, signs) -> np.ndarray:
    """R^T y for every row: the key a rotated row stands for (y @ R)."""
    return np.asarray(y, dtype=np.float64) @ rotation(signs)
