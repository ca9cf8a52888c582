"""Seeded generator for the drafter's weights and round inputs.

Shapes follow the Kolibri-1 block-drafter model card (section "Architecture"):
three tapped 2560-wide states fused 7680->2560, the 5120->2560 context-row
projection, 4 layers of hidden 2560 with 20 heads of 128 and a SwiGLU FFN of
6144, rank-256 predecessor and spine adapters, and a 60,614-row draft
vocabulary over a 131,072-row embedding/head table.

Formats (model card, "Architecture", serving paragraph): the body is block-FP8,
e4m3 values with one fp32 scale per row and 64 inputs; the head slice is NVFP4:
e2m1 values, one e4m3 scale per 16 inputs and one fp32 tensor scale.

Every tensor has its own generator, seeded from (base seed, tensor name[, stream]),
so any tensor, or one stream's inputs, can be regenerated alone. Big tensors are
drawn with torch on the requested device; the values are whatever that device's
generator yields, and both sides of a parity check consume the same bytes.
"""
from __future__ import annotations

import dataclasses
import zlib

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Dims:
    hidden: int = 2560
    heads: int = 20
    head_dim: int = 128
    ffn: int = 6144
    layers: int = 4
    block: int = 4
    rank: int = 256
    window: int = 2048
    capacity: int = 2048
    draft_vocab: int = 60614
    full_vocab: int = 131072
    taps: int = 3
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6


FULL = Dims()
# A small model with the same structure, for fast oracle checks. Every inner
# dimension stays a multiple of 64 so block-FP8 rows split into whole blocks.
TINY = Dims(hidden=128, heads=2, head_dim=64, ffn=192, layers=4, block=4, rank=64,
            window=32, capacity=32, draft_vocab=300, full_vocab=1000)


# The five synthetic workloads (stream count, context-length law, adapter state).
CONFIGS = [
    dict(name="B1", streams=1, lens=("const", 2048), model="A", ingest=0),
    dict(name="B4", streams=4, lens=("const", 2048), model="A", ingest=0),
    dict(name="B16-ragged", streams=16, lens=("uniform", 256, 4096), model="B", ingest=0),
    dict(name="B64-ingest", streams=64, lens=("const", 2043), model="A", ingest=5),
    dict(name="B256-ragged", streams=256, lens=("uniform", 512, 2048), model="A", ingest=0),
]


def _seed(*parts) -> int:
    ss = np.random.SeedSequence([int(p) if not isinstance(p, str) else zlib.crc32(p.encode())
                                 for p in parts])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def _normal(shape, std, device, *parts) -> torch.Tensor:
    return torch.randn(shape, generator=_gen(device, *parts), device=device,
                       dtype=torch.float32) * std


def bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """Round to bf16 (round-to-nearest-even, torch's cast) and return the bits."""
    return x.to(torch.bfloat16).view(torch.int16)


# ----------------------------------------------------------------------------
# Load-time quantisers. The round consumes their output bytes; it never
# quantises anything itself.
# ----------------------------------------------------------------------------

def quant_block_fp8(w: torch.Tensor):
    """Block-FP8: per row and per 64 inputs, s = amax/448 (1 if the block is 0)
    and q = e4m3(w/s) rounded to nearest even by torch's float8_e4m3fn cast."""
    rows, cols = w.shape
    assert cols % 64 == 0
    wb = w.float().reshape(rows, cols // 64, 64)
    amax = wb.abs().amax(-1)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (wb / s[..., None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(rows, cols).contiguous(), s.contiguous()


def e2m1_codes(y: torch.Tensor) -> torch.Tensor:
    """Round to the nearest e2m1 value {0,.5,1,1.5,2,3,4,6}, ties to the even
    mantissa, saturating at 6; returns 4-bit codes (bit 3 = sign)."""
    a = y.abs()
    code = ((a > 0.25).to(torch.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
            + (a > 2.5) + (a >= 3.5) + (a > 5.0)).to(torch.uint8)
    sign = ((y < 0) & (code > 0)).to(torch.uint8) << 3
    return code | sign


def quant_nvfp4(w: torch.Tensor, g: float | None = None):
    """NVFP4 with a tensor scale g (default amax/(6*448)), an e4m3 scale per 16
    inputs s_b = e4m3(amax_b/(6g)) and e2m1 codes of w/(s_b*g). Two codes per
    byte, the even column in the low nibble. Returns (q4, s4 codes, g)."""
    rows, cols = w.shape
    assert cols % 16 == 0
    w = w.float()
    if g is None:
        amax = float(w.abs().max())
        g = amax / (6.0 * 448.0) if amax > 0 else 1.0
    g32 = torch.tensor(g, dtype=torch.float32, device=w.device)
    wb = w.reshape(rows, cols // 16, 16)
    amax_b = wb.abs().amax(-1)
    s = (amax_b / (6.0 * g32)).clamp(max=448.0).to(torch.float8_e4m3fn)
    denom = s.float() * g32
    y = torch.where(denom[..., None] > 0, wb / torch.where(denom > 0, denom, 1.0)[..., None],
                    torch.zeros_like(wb))
    codes = e2m1_codes(y).reshape(rows, cols)
    q4 = (codes[:, 0::2] | (codes[:, 1::2] << 4)).contiguous()
    return q4, s.view(torch.uint8).contiguous(), float(g32)


# ----------------------------------------------------------------------------
# Model
# ----------------------------------------------------------------------------

def _fp8(model, name, rows, cols, device, base, zero=False, body="fp8"):
    """One body matrix, N(0, 0.02) (or zero), in the body format: block-FP8
    (.q, .s), NVFP4 (.q4, .s4, .g, one tensor scale per matrix) or bf16
    (.bf16, round to nearest even). Every format quantises the same draws."""
    if zero:
        w = torch.zeros(rows, cols, device=device)
    else:
        w = _normal((rows, cols), 0.02, device, base, name)
    if body == "nvfp4":
        model[name + ".q4"], model[name + ".s4"], model[name + ".g"] = quant_nvfp4(w)
    elif body == "bf16":
        model[name + ".bf16"] = w.to(torch.bfloat16).contiguous()
    else:
        q, s = quant_block_fp8(w)
        model[name + ".q"] = q
        model[name + ".s"] = s


def make_model(dims: Dims = FULL, variant: str = "A", device="cpu", base: int = 0,
               head: str = "nvfp4", body: str = "fp8"):
    """Synthetic drafter weights.

    variant "A": predecessor and spine output projections U are zero (the
    adapters are zero-initialised, so they add nothing), A/B random.
    variant "B": every adapter matrix N(0, 0.02), so both adapters are active.
    variant "C": as "B" with RMSNorm gains 1 + N(0, 0.1) instead of 1.
    All other matrices N(0, 0.02) -> block-FP8. The mask row is N(0, 0.02).
    The embedding/head table is N(0, 0.02) rounded to bf16; the head is the
    NVFP4 quantisation of its rows at the (sorted) draft vocabulary.
    kv_rot_signs: int8 [layers][head_dim], each +1 or -1 with probability 1/2
    (the random signs of a rotated 4-bit K/V cache).
    head="bf16": the head slice is also given unquantised, head_bf16 = the
    table's bf16 rows at the draft vocabulary (head_format "bf16");
    head="fp8": also as block-FP8 of those rows (head_fp8.q / .s).
    body="nvfp4" / "bf16": the body matrices in that format instead of
    block-FP8 (body_format), quantised from the same draws.
    """
    assert variant in ("A", "B", "C") and body in ("fp8", "nvfp4", "bf16")
    H, F, r, L = dims.hidden, dims.ffn, dims.rank, dims.layers
    zero_u = variant == "A"
    m: dict = {"dims": dims, "variant": variant, "body_format": body}
    _fp8(m, "fuse", H, dims.taps * H, device, base, body=body)
    _fp8(m, "fc", H, 2 * H, device, base, body=body)
    _fp8(m, "pred_a", r, H, device, base, body=body)
    _fp8(m, "pred_b", r, H, device, base, body=body)
    _fp8(m, "pred_u", H, r, device, base, zero=zero_u, body=body)
    m["mask"] = _normal((H,), 0.02, device, base, "mask")

    def gain(name):
        if variant == "C":
            return 1.0 + _normal((H,), 0.1, device, base, name)
        return torch.ones(H, device=device)

    for l in range(L):
        p = f"layers.{l}."
        m[p + "attn_norm"] = gain(p + "attn_norm")
        m[p + "ffn_norm"] = gain(p + "ffn_norm")
        for nm, (ro, co) in dict(wq=(H, H), wk=(H, H), wv=(H, H), wo=(H, H),
                                 w_gate=(F, H), w_up=(F, H), w_down=(H, F)).items():
            _fp8(m, p + nm, ro, co, device, base, body=body)
        if l >= 1:
            sp = f"spine.{l}."
            m[sp + "norm"] = gain(sp + "norm")
            _fp8(m, sp + "a", r, H, device, base, body=body)
            _fp8(m, sp + "u", H, r, device, base, zero=zero_u, body=body)
    m["final_norm"] = gain("final_norm")

    table = _normal((dims.full_vocab, H), 0.02, device, base, "table").to(torch.bfloat16)
    perm = torch.randperm(dims.full_vocab, generator=_gen("cpu", base, "vocab"))
    vocab = torch.sort(perm[: dims.draft_vocab]).values.to(torch.int32)
    m["table"] = table
    m["vocab"] = vocab.to(device)
    q4, s4, g = quant_nvfp4(table[vocab.to(device).long()].float())
    m["head.q4"], m["head.s4"], m["head.g"] = q4, s4, g
    # one random sign per head dimension and layer, for a rotated 4-bit cache
    signs = torch.randint(0, 2, (L, dims.head_dim), generator=_gen("cpu", base, "kv_rot_signs"))
    m["kv_rot_signs"] = (1 - 2 * signs).to(torch.int8).to(device)
    assert head in ("nvfp4", "bf16", "fp8")
    m["head_format"] = head
    if head == "bf16":
        m["head_bf16"] = table[vocab.to(device).long()].contiguous()
    if head == "fp8":
        m["head_fp8.q"], m["head_fp8.s"] = quant_block_fp8(table[vocab.to(device).long()].float())
    return m


def model_bytes(dims: Dims = FULL, body: str = "fp8"):
    """Bytes the round reads for weights: block-FP8 body (1 B per value + 4 B
    per 64 values; NVFP4: 0.5 B per value + 1 B per 16 + 4 B per matrix;
    bf16: 2 B per value), NVFP4 head (0.5 B per value + 1 B per 16 + 4 B),
    fp32 vectors (mask row and gains)."""
    H, F, r, L, T = dims.hidden, dims.ffn, dims.rank, dims.layers, dims.taps
    vals = H * T * H + H * 2 * H + 2 * r * H + H * r
    vals += L * (4 * H * H + 3 * F * H)
    vals += (L - 1) * 2 * r * H
    mats = 5 + 7 * L + 2 * (L - 1)
    if body == "nvfp4":
        body_b = vals // 2 + vals // 16 + 4 * mats
    elif body == "bf16":
        body_b = 2 * vals
    else:
        body_b = vals + vals // 64 * 4
    head = dims.draft_vocab * H // 2 + dims.draft_vocab * H // 16 + 4
    vectors = 4 * H * (1 + 2 * L + (L - 1) + 1)
    return dict(body=body_b, head=head, vectors=vectors)


# ----------------------------------------------------------------------------
# Round inputs
# ----------------------------------------------------------------------------

def _rms_normal(shape, device, *parts):
    x = _normal(shape, 1.0, device, *parts)
    return x / x.pow(2).mean(-1, keepdim=True).sqrt()


def make_inputs(cfg: dict, dims: Dims = FULL, device="cpu", base: int | None = None,
                poison: bool = False, vocab: torch.Tensor | None = None, streams=None,
                lens_override=None, kv: str = "bf16"):
    """Round inputs for one workload.

    Each stream's tensors are seeded by (base, name, stream), so stream b's
    inputs are the same whatever the batch around it.
      taps   bf16 [B][3][H]: N(0,1) per H-vector, divided by its RMS
      anchor int32 [B], pred int32 [B][3]: uniform over the draft vocabulary
      lens   int32 [B]: tokens seen; rows at positions [len-n, len) with
             n = min(len, window) are visible, stored at slot pos % capacity
      k, v   per layer bf16 [B][heads][capacity][head_dim]: N(0,1) at visible
             slots; NaN elsewhere when poison=True (out-of-window reads show up)
      ingest (when cfg["ingest"] > 0): taps [B][n][3][H] and next ids [B][n]
    lens_override: explicit per-stream lengths instead of the config's law.
    kv="int4": the cache holds 4-bit codes instead (see _int4_cache); then
      k, v are uint8 [B][heads][capacity][head_dim/2] and k_so, v_so are
      fp16 bits uint16 [B][heads][capacity][2] (scale, offset); invisible
      slots get NaN scale and offset when poison=True.
    """
    if base is None:
        base = 100 + CONFIGS.index(cfg) if cfg in CONFIGS else 100
    B = cfg["streams"] if streams is None else streams
    if lens_override is not None:
        B = len(lens_override)
    if vocab is None:
        perm = torch.randperm(dims.full_vocab, generator=_gen("cpu", 0, "vocab"))
        vocab = torch.sort(perm[: dims.draft_vocab]).values.to(torch.int32)
    vocab_cpu = vocab.cpu().long()
    H, NH, D, C = dims.hidden, dims.heads, dims.head_dim, dims.capacity
    inp: dict = {"dims": dims, "streams": B}

    def ids(shape, *parts):
        g = _gen("cpu", base, *parts)
        return vocab_cpu[torch.randint(0, dims.draft_vocab, shape, generator=g)].to(torch.int32)

    taps, anchor, pred, lens = [], [], [], []
    mode = cfg["lens"]
    for b in range(B):
        taps.append(_rms_normal((dims.taps, H), device, base, "taps", b).to(torch.bfloat16))
        anchor.append(ids((1,), "anchor", b))
        pred.append(ids((dims.block - 1,), "pred", b))
        if lens_override is not None:
            lens.append(int(lens_override[b]))
        elif mode[0] == "const":
            lens.append(int(mode[1]))
        else:
            g = _gen("cpu", base, "len", b)
            lens.append(int(torch.randint(mode[1], mode[2] + 1, (1,), generator=g)))
    inp["taps"] = torch.stack(taps)
    inp["anchor"] = torch.cat(anchor).to(device)
    inp["pred"] = torch.stack(pred).to(device)
    inp["lens"] = torch.tensor(lens, dtype=torch.int32, device=device)

    if kv == "int4":
        _int4_cache(inp, dims, B, lens, device, base, poison)
        ks = vs = None
    else:
        assert kv == "bf16"
        ks, vs = _bf16_cache(dims, B, lens, device, base, poison)
    if ks is not None:
        inp["k"], inp["v"] = ks, vs

    n_new = cfg.get("ingest", 0)
    if n_new:
        inp["ingest_taps"] = torch.stack([
            _rms_normal((n_new, dims.taps, H), device, base, "itaps", b).to(torch.bfloat16)
            for b in range(B)])
        inp["ingest_ids"] = torch.stack([ids((n_new,), "iids", b) for b in range(B)]).to(device)
    return inp


def _visible_mask(dims, length, C):
    n = min(length, dims.window)
    pos = torch.arange(length - n, length)
    vis = torch.zeros(C, dtype=torch.bool)
    vis[pos % C] = True
    return vis


def _bf16_cache(dims, B, lens, device, base, poison):
    NH, D, C = dims.heads, dims.head_dim, dims.capacity
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16, device=device)
    ks, vs = [], []
    for l in range(dims.layers):
        for name, store in (("k", ks), ("v", vs)):
            t = torch.empty((B, NH, C, D), dtype=torch.bfloat16, device=device)
            for b in range(B):
                x = _normal((NH, C, D), 1.0, device, base, f"{name}{l}", b).to(torch.bfloat16)
                if poison:
                    x[:, ~_visible_mask(dims, lens[b], C).to(device)] = nan
                t[b] = x
            store.append(t)
    return ks, vs


def _int4_cache(inp, dims, B, lens, device, base, poison):
    """A 4-bit cache drawn directly in its stored form (no quantiser runs
    here): per element a code round(7.5 + 2.5 z) clamped to 0..15 (z ~ N(0,1)),
    two per byte with the even dimension in the low nibble; per (stream, head,
    slot) an fp16 scale ~ U(0.25, 0.45) and an fp16 offset of
    -7.5 * scale + N(0, 0.1), so scale * code + offset is roughly N(0, 0.8)."""
    NH, D, C = dims.heads, dims.head_dim, dims.capacity
    nan16 = 0x7E00
    out = {"k": [], "v": [], "k_so": [], "v_so": []}
    for l in range(dims.layers):
        for name in ("k", "v"):
            codes = torch.empty((B, NH, C, D // 2), dtype=torch.uint8, device=device)
            so = torch.empty((B, NH, C, 2), dtype=torch.int16, device=device)
            for b in range(B):
                z = _normal((NH, C, D), 1.0, device, base, f"{name}{l}q", b)
                c = (7.5 + 2.5 * z).round().clamp(0, 15).to(torch.uint8)
                codes[b] = c[..., 0::2] | (c[..., 1::2] << 4)
                g = _gen(device, base, f"{name}{l}so", b)
                sc = (0.25 + 0.2 * torch.rand((NH, C), generator=g, device=device)).to(torch.float16)
                off = (-7.5 * sc.float()
                       + 0.1 * torch.randn((NH, C), generator=g, device=device)).to(torch.float16)
                pair = torch.stack([sc.view(torch.int16), off.view(torch.int16)], dim=-1)
                if poison:
                    pair[:, ~_visible_mask(dims, lens[b], C).to(device)] = nan16
                so[b] = pair
            out[name].append(codes)
            out[name + "_so"].append(so)
    inp.update(out)
    inp["kv_format"] = "int4"


# ----------------------------------------------------------------------------
# numpy views for the oracle (bit patterns only; no arithmetic)
# ----------------------------------------------------------------------------

def _np(t):
    if isinstance(t, torch.Tensor):
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()
    return t


def to_numpy_model(m: dict) -> dict:
    return {k: (_np(v) if isinstance(v, torch.Tensor) else v) for k, v in m.items()}


def to_numpy_inputs(inp: dict, streams=None) -> dict:
    """numpy copy of the inputs, optionally only a subset of streams."""
    sel = slice(None) if streams is None else list(streams)
    out = {"dims": inp["dims"]}
    for k in ("taps", "anchor", "pred", "lens", "ingest_taps", "ingest_ids"):
        if k in inp:
            out[k] = _np(inp[k][sel])
    out["k"] = [_np(t[sel]) for t in inp["k"]]
    out["v"] = [_np(t[sel]) for t in inp["v"]]
    if inp.get("kv_format") == "int4":
        out["kv_format"] = "int4"
        out["k_so"] = [_np(t[sel]).view(np.uint16) for t in inp["k_so"]]
        out["v_so"] = [_np(t[sel]).view(np.uint16) for t in inp["v_so"]]
    out["streams"] = len(out["lens"])
    return out
