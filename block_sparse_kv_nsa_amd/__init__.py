"""Block-sparse long-context decode attention for MI355X (gfx950).

The work is done by ``libnsa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/nsa.h``); this package is its ctypes binding.  Importing
it without the built library raises ImportError: there is no fallback path.
"""

from ._abi import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    NSA_BF16,
    NSA_ERR_HIP,
    NSA_ERR_INVALID_ARGUMENT,
    NSA_ERR_STEP_EXPIRED,
    NSA_ERR_UNSUPPORTED,
    NSA_ERR_WORKSPACE_TOO_SMALL,
    NSA_F32,
    NSA_OK,
    NSA_SCORE_FORECAST_RAW,
    NSA_SCORE_FORECAST_WINDOW,
    NSA_SCORE_GROUP_SOFTMAX,
    DecodeParams,
    NsaError,
    PrefillParams,
    SelectParams,
    Shape,
    StepGrid,
    load,
    nsa_abi_version,
    nsa_decode_step,
    nsa_decode_step_grid,
    nsa_decode_step_noalloc,
    nsa_decode_step_status,
    nsa_debug_checks,
    nsa_debug_error,
    nsa_decode_step_workspace_bytes,
    nsa_decode_workspace_bytes,
    nsa_last_error,
    nsa_residency_diff,
    nsa_s2o_attend,
    nsa_s2o_index,
    nsa_s2o_workspace_bytes,
    nsa_select_blocks,
    nsa_select_workspace_bytes,
    nsa_sparse_decode,
    nsa_sparse_decode_biased,
    nsa_status_string,
    nsa_update_block_reps,
)

load()

from .layer import SparseDecodeLayer  # noqa: E402,F401
