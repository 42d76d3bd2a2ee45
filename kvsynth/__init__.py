"""Seeded synthetic workloads shared by the oracle-based tests and the bench.

Holds input shapes and input draws only; no scoring, selection or eviction
arithmetic lives here.
"""

from .configs import (LoreConfig, H2OConfig, RefreshConfig, TINY, MISTRAL_16K, LLAMA_128K,
                      QWEN_14B_BATCH, OPT30B_H2O, QWEN7B_REFRESH, LORE_CONFIGS, H2O_CONFIGS)
from .gen import (lore_inputs, h2o_inputs, trajectory_token_stats, future_queries,
                  refresh_inputs, TORCH_DTYPES)

__all__ = ["LoreConfig", "H2OConfig", "RefreshConfig", "QWEN7B_REFRESH", "refresh_inputs", "TINY", "MISTRAL_16K", "LLAMA_128K",
           "QWEN_14B_BATCH", "OPT30B_H2O", "LORE_CONFIGS", "H2O_CONFIGS",
           "lore_inputs", "h2o_inputs", "trajectory_token_stats", "future_queries",
           "TORCH_DTYPES"]
