"""fp64 CPU oracle of one Kolibri-1 block-drafter round.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The library under
``block_draft_model_amd`` never calls it and shares no code with it.
"""
from . import kv_int4
from .copy_draft import PauseGuard, copy_draft
from .kdraft_oracle import (decode_e4m3, decode_e2m1, decode_bf16, round_bf16,
                            block_fp8, nvfp4, rmsnorm, silu, rope, attention,
                            OracleModel, oracle_round, oracle_round_depth, oracle_ingest,
                            top2_gap)

__all__ = ["kv_int4", "copy_draft", "PauseGuard", "decode_e4m3", "decode_e2m1", "decode_bf16", "round_bf16", "block_fp8", "nvfp4",
           "rmsnorm", "silu", "rope", "attention", "OracleModel", "oracle_round",
           "oracle_round_depth", "oracle_ingest", "top2_gap"]
