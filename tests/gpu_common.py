"""Shared pieces of the GPU tests: one library context per synthetic model,
seeded inputs on the device, and the acceptance rule against the oracle.

Acceptance (per block row): relative L2 error of the logits <= 1e-2, and the
draft id equal to the oracle's wherever the oracle's top-1/top-2 logit gap
exceeds 1e-2 (where the gap is smaller, either of the near-tied ids is a
correct draft).
"""
from __future__ import annotations

import sys
import time

import numpy as np
import pytest
import torch

import oracle
import synth
from block_draft_model_amd import kdraft

REL_L2_MAX = 1e-2
GAP_MIN = 1e-2


def log(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


class Harness:
    """A synthetic model on the GPU, loaded into one kd_ctx, plus its oracle."""

    def __init__(self, variant: str, max_streams: int = 256, window: int = 2048,
                 head: str = "nvfp4", body: str = "fp8"):
        t0 = time.time()
        self.variant = variant
        self.head = head
        self.body = body
        self.model = synth.make_model(synth.FULL, variant, device="cuda", head=head, body=body)
        quant = {"nvfp4": kdraft.KD_QUANT_NVFP4, "bf16": kdraft.KD_QUANT_BF16,
                 "fp8": kdraft.KD_QUANT_FP8_BLOCK64}
        self.drafter = kdraft.Drafter(max_streams=max_streams, window=window, head_quant=quant[head],
                                      body_quant=quant[body])
        self.drafter.load_weights(self.model)
        self._oracle = None
        log(f"model {variant} ready in {time.time() - t0:.1f}s")

    @property
    def oracle(self):
        if self._oracle is None:
            t0 = time.time()
            self._oracle = oracle.OracleModel(synth.to_numpy_model(self.model))
            log(f"oracle model {self.variant} decoded in {time.time() - t0:.1f}s")
        return self._oracle

    def inputs(self, cfg, **kw):
        kw.setdefault("poison", True)
        return synth.make_inputs(cfg, synth.FULL, device="cuda", vocab=self.model["vocab"], **kw)

    @staticmethod
    def kv(inp):
        if inp.get("kv_format") == "int4":
            return kdraft.kv_struct_int4(inp["k"], inp["v"], inp["k_so"], inp["v_so"])
        return kdraft.kv_struct(inp["k"], inp["v"])

    def run(self, inp, logits=True):
        B = inp["streams"]
        kv = self.kv(inp)
        ids = torch.full((B, 4), -7, dtype=torch.int32, device="cuda")
        lg = torch.full((B, 4, synth.FULL.draft_vocab), float("nan"), device="cuda") if logits else None
        self.drafter.round(B, inp["taps"], inp["anchor"], inp["pred"], kv, inp["lens"], ids, lg)
        torch.cuda.synchronize()
        return (lg.cpu().numpy().astype(np.float64) if logits else None), ids.cpu().numpy()

    def ingest(self, inp):
        B = inp["streams"]
        kv = self.kv(inp)
        n = inp["ingest_ids"].shape[1]
        self.drafter.ingest(B, n, inp["ingest_taps"], inp["ingest_ids"], kv, inp["lens"])
        torch.cuda.synchronize()


def compare(gpu_logits, gpu_ids, ref_logits, ref_ids, vocab, label=""):
    g = gpu_logits.reshape(-1, gpu_logits.shape[-1])
    r = ref_logits.reshape(-1, ref_logits.shape[-1])
    rel = np.linalg.norm(g - r, axis=1) / np.linalg.norm(r, axis=1)
    gap = oracle.top2_gap(r)
    gated = gap > GAP_MIN
    gi, ri = gpu_ids.reshape(-1), ref_ids.reshape(-1)
    mism = int(np.sum((gi != ri) & gated))
    exempt_diff = int(np.sum((gi != ri) & ~gated))
    stats = dict(rows=len(rel), max_rel_l2=float(rel.max()), gated=int(gated.sum()),
                 mismatches=mism, exempt_differing=exempt_diff, min_gap=float(gap.min()))
    log(label, stats)
    assert np.all(np.isfinite(g)), "non-finite GPU logits"
    assert rel.max() <= REL_L2_MAX, stats
    assert mism == 0, stats
    # where ids differ on a near-tie row, the GPU's id is one of the oracle's top two
    vocab = np.asarray(vocab)
    for k in np.nonzero((gi != ri) & ~gated)[0]:
        top2 = vocab[np.argsort(-r[k])[:2]]
        assert gi[k] in set(int(x) for x in top2), (k, gi[k], top2)
    return stats
