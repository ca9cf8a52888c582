"""Seeded synthetic inputs for the Kolibri-1 block-drafter round.

This package is shared by the oracle's tests, the GPU tests and the benchmark.
It only *produces* inputs: random weights (quantised to the load-time formats),
tapped states, ids, context lengths and context K/V. It holds none of the
round's arithmetic; both the oracle and the HIP library decode what it writes
on their own.
"""
from .gen import (Dims, FULL, TINY, CONFIGS, make_model, make_inputs,
                  quant_block_fp8, quant_nvfp4, e2m1_codes, bf16_bits, to_numpy_model,
                  to_numpy_inputs, model_bytes)

__all__ = ["Dims", "FULL", "TINY", "CONFIGS", "make_model", "make_inputs",
           "quant_block_fp8", "quant_nvfp4", "e2m1_codes", "bf16_bits",
           "to_numpy_model", "to_numpy_inputs", "model_bytes"]
