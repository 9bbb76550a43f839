"""Seeded synthetic inputs for MSA decode (shared by the tests, the oracle
checks and bench.py). Holds no part of the decode arithmetic."""
from .gen import (Workload, make_workload, make_config, make_new_tokens, small_cases, ragged_lengths,
                  CONFIG_NAMES, KV_BF16, KV_NVFP4, IDX_BF16, IDX_FP8, IDX_NVFP4)

__all__ = ["Workload", "make_workload", "make_config", "make_new_tokens", "small_cases", "ragged_lengths",
           "CONFIG_NAMES", "KV_BF16", "KV_NVFP4", "IDX_BF16", "IDX_FP8", "IDX_NVFP4"]
