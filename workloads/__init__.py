"""Seeded synthetic inputs for block-sparse decode attention.

This package only draws and lays out input tensors.  It holds none of the
method's arithmetic (no block representatives, scores, selection or
attention): both the CPU oracle and the GPU path consume what it produces.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    Batch,
    Config,
    RowInputs,
    bf16_bits_to_f32,
    block_table,
    build_batch,
    config,
    f32_to_bf16_bits,
    forecast_row,
    forecasts,
    key_centre,
    planted_blocks,
    queries,
    query_row,
    row_inputs,
    scatter_row,
    storage_dtype,
    stored_to_f64,
)
from .prefill import (  # noqa: F401
    PREFILL_CONFIGS,
    PrefillBatch,
    PrefillConfig,
    build_prefill,
    kv_row,
    prefill_config,
    prefill_table,
    q_row,
)
