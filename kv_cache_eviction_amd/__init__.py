"""KV-cache scoring and eviction on MI355X (gfx950).

The computation lives in libkvscore.so (hand-written HIP kernels behind the C
ABI of include/kvscore.h).  This package is its thin binding: the entry
points keep the C names and take torch device tensors; ``LoreEviction`` wires
the LORE-KV calls of one layer together with preallocated buffers.
"""

from ._lib import (KvsError, LoreDesc, H2ODesc, load, last_error, lore_desc, h2o_desc,
                   kvs_lore_workspace_bytes, kvs_topb_workspace_bytes, kvscore_probs, kvscore_deletion,
                   kvscore_baseline_scores, kvscore_reliability_weights, RELIABILITY_E,
                   kvs_fidelity_workspace_bytes, kvscore_output_fidelity,
                   kvscore_counter_causal,
                   kvs_refresh_workspace_bytes, kvscore_refresh,
                   RELIABILITY_D, kvscore_topb_select, kvscore_topb_select_noalloc, kvscore_retention_shift,
                   kv_compact,
                   kvs_h2o_workspace_bytes,
                   kvscore_h2o_accumulate, KVS_F32, KVS_BF16, KVS_F16, KVS_H2O_PREFILL,
                   KVS_H2O_DECODE, KVS_BASELINE_WINDOW, KVS_BASELINE_TOVA, KVS_MASK_NONE,
                   KVS_MASK_WINDOW_CAUSAL, KVS_MASK_CAUSAL, KVS_MASK_SLOTS, DTYPE_CODE, EXPORTS, LIB_PATH, kvs_timing_enable,
                   kvs_measure_peaks,
                   kvs_timing_reset, kvs_timing_records)
from .evict import LoreEviction, H2OCache

__all__ = ["KvsError", "LoreDesc", "H2ODesc", "load", "last_error", "lore_desc", "h2o_desc",
           "kvs_lore_workspace_bytes", "kvs_topb_workspace_bytes", "kvscore_probs", "kvscore_deletion",
           "kvscore_baseline_scores", "kvscore_reliability_weights", "RELIABILITY_E",
           "kvs_fidelity_workspace_bytes", "kvscore_output_fidelity",
           "kvscore_counter_causal",
           "kvs_refresh_workspace_bytes", "kvscore_refresh",
           "RELIABILITY_D", "KVS_BASELINE_WINDOW", "KVS_BASELINE_TOVA", "kvscore_topb_select", "kvscore_topb_select_noalloc", "kvscore_retention_shift", "kv_compact", "kvs_h2o_workspace_bytes",
           "kvscore_h2o_accumulate", "KVS_F32", "KVS_BF16", "KVS_F16", "KVS_H2O_PREFILL",
           "KVS_H2O_DECODE", "KVS_MASK_NONE", "KVS_MASK_WINDOW_CAUSAL", "KVS_MASK_CAUSAL",
           "KVS_MASK_SLOTS", "DTYPE_CODE", "EXPORTS", "LIB_PATH", "LoreEviction", "H2OCache",
           "kvs_timing_enable", "kvs_timing_reset", "kvs_timing_records", "kvs_measure_peaks"]
