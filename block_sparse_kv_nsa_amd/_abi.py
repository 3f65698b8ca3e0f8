"""ctypes binding of libnsa.so: the C ABI declared in include/nsa.h.

Argument marshalling only.  Tensors are passed by their device pointer,
streams by their HIP handle; every computation happens in the library's
kernels.  torch is imported before the library is loaded so that libnsa's
``libamdhip64.so.7`` resolves to the HIP runtime torch already loaded (one
runtime per process, so torch's streams and allocations are valid here).
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede loading libnsa; see module docstring)

# NSA_LIB_PATH selects another build of the library (e.g. a debug build)
LIB_PATH = os.environ.get("NSA_LIB_PATH") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libnsa.so")

NSA_OK = 0
NSA_ERR_INVALID_ARGUMENT = 1
NSA_ERR_UNSUPPORTED = 2
NSA_ERR_WORKSPACE_TOO_SMALL = 3
NSA_ERR_HIP = 4
NSA_ERR_STEP_EXPIRED = 5

NSA_F32 = 0
NSA_BF16 = 1

NSA_SCORE_GROUP_SOFTMAX = 0
NSA_SCORE_FORECAST_RAW = 1
NSA_SCORE_FORECAST_WINDOW = 2

EXPORTS = (
    "nsa_update_block_reps",
    "nsa_select_workspace_bytes",
    "nsa_select_blocks",
    "nsa_decode_workspace_bytes",
    "nsa_sparse_decode",
    "nsa_sparse_decode_biased",
    "nsa_decode_step_workspace_bytes",
    "nsa_decode_step",
    "nsa_decode_step_noalloc",
    "nsa_decode_step_status",
    "nsa_decode_step_grid",
    "nsa_residency_diff",
    "nsa_s2o_workspace_bytes",
    "nsa_s2o_index",
    "nsa_s2o_attend",
    "nsa_debug_checks",
    "nsa_debug_error",
    "nsa_status_string",
    "nsa_last_error",
    "nsa_abi_version",
)


class NsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("sub_block", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_phys_blocks", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]

    @classmethod
    def make(cls, batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
             num_phys_blocks, dtype, softmax_scale=0.0, block_size=64, sub_block=16):
        return cls(batch, num_q_heads, num_kv_heads, head_dim, block_size, sub_block,
                   max_blocks_per_seq, num_phys_blocks, dtype, softmax_scale)


class SelectParams(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("k_e", ctypes.c_int32),
        ("ordered", ctypes.c_int32),
    ]


class StepGrid(ctypes.Structure):
    _fields_ = [
        ("workgroups", ctypes.c_int32),
        ("scorers_per_row", ctypes.c_int32),
        ("attenders_per_row", ctypes.c_int32),
        ("rows_at_once", ctypes.c_int32),
        ("reps_per_scorer", ctypes.c_int32),
    ]


class DecodeParams(ctypes.Structure):
    _fields_ = [
        ("max_selected", ctypes.c_int32),
        ("early_stop", ctypes.c_int32),
        ("tau", ctypes.c_float),
    ]


class PrefillParams(ctypes.Structure):
    _fields_ = [
        ("segment", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("tau", ctypes.c_float),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load libnsa.so (raises ImportError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python block_sparse_kv_nsa_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    P = ctypes.POINTER
    lib.nsa_update_block_reps.argtypes = [P(Shape), vp, vp, vp, vp, vp, i32, vp, vp, vp]
    lib.nsa_update_block_reps.restype = i32
    lib.nsa_select_workspace_bytes.argtypes = [P(Shape), P(SelectParams), i32, P(sz)]
    lib.nsa_select_workspace_bytes.restype = i32
    lib.nsa_select_blocks.argtypes = [P(Shape), P(SelectParams), vp, vp, vp, vp, i32, vp, vp,
                                      vp, vp, vp, sz, vp]
    lib.nsa_select_blocks.restype = i32
    lib.nsa_decode_workspace_bytes.argtypes = [P(Shape), P(DecodeParams), P(sz)]
    lib.nsa_decode_workspace_bytes.restype = i32
    lib.nsa_sparse_decode.argtypes = [P(Shape), P(DecodeParams), vp, vp, vp, vp, vp, vp, vp,
                                      vp, vp, vp, sz, vp]
    lib.nsa_sparse_decode.restype = i32
    lib.nsa_sparse_decode_biased.argtypes = [P(Shape), P(DecodeParams), vp, vp, vp, vp, vp, vp, vp,
                                             vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.nsa_sparse_decode_biased.restype = i32
    lib.nsa_decode_step_workspace_bytes.argtypes = [P(Shape), P(SelectParams), i32, P(sz)]
    lib.nsa_decode_step_workspace_bytes.restype = i32
    lib.nsa_decode_step.argtypes = [P(Shape), P(SelectParams), vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                    vp, vp, vp, vp, vp, vp, sz, vp]
    lib.nsa_decode_step.restype = i32
    lib.nsa_decode_step_noalloc.argtypes = [P(Shape), P(SelectParams), vp, vp, vp, vp, vp, vp, vp,
                                            vp, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.nsa_decode_step_noalloc.restype = i32
    lib.nsa_decode_step_status.argtypes = [vp, sz, i32, vp]
    lib.nsa_decode_step_status.restype = i32
    lib.nsa_residency_diff.argtypes = [P(Shape), i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.nsa_residency_diff.restype = i32
    lib.nsa_s2o_workspace_bytes.argtypes = [P(Shape), P(PrefillParams), P(sz)]
    lib.nsa_s2o_workspace_bytes.restype = i32
    lib.nsa_s2o_index.argtypes = [P(Shape), P(PrefillParams), vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.nsa_s2o_index.restype = i32
    lib.nsa_s2o_attend.argtypes = [P(Shape), P(PrefillParams), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                   vp, sz, vp]
    lib.nsa_s2o_attend.restype = i32
    lib.nsa_decode_step_grid.argtypes = [P(Shape), P(SelectParams), i32, i32, P(StepGrid)]
    lib.nsa_decode_step_grid.restype = i32
    lib.nsa_debug_checks.argtypes = []
    lib.nsa_debug_checks.restype = i32
    lib.nsa_debug_error.argtypes = [P(ctypes.c_uint32), i32]
    lib.nsa_debug_error.restype = i32
    lib.nsa_status_string.argtypes = [i32]
    lib.nsa_status_string.restype = ctypes.c_char_p
    lib.nsa_last_error.argtypes = []
    lib.nsa_last_error.restype = ctypes.c_char_p
    lib.nsa_abi_version.argtypes = []
    lib.nsa_abi_version.restype = i32
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return ctypes.c_void_p(x)
    return ctypes.c_void_p(x.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream
                               if torch.cuda.is_available() else 0)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, name: str) -> None:
    if status != NSA_OK:
        lib = load()
        raise NsaError(status, f"{name}: {lib.nsa_status_string(status).decode()}: "
                               f"{lib.nsa_last_error().decode()}")


def nsa_status_string(status: int) -> str:
    return load().nsa_status_string(status).decode()


def nsa_last_error() -> str:
    return load().nsa_last_error().decode()


def nsa_abi_version() -> int:
    return load().nsa_abi_version()


def nsa_update_block_reps(shape: Shape, k_pool, block_table, evict_logits, first_block,
                          num_blocks, max_num_blocks: int, reps, evict_block_score,
                          stream=None) -> None:
    st = load().nsa_update_block_reps(ctypes.byref(shape), _ptr(k_pool), _ptr(block_table),
                                      _ptr(evict_logits), _ptr(first_block), _ptr(num_blocks),
                                      int(max_num_blocks), _ptr(reps), _ptr(evict_block_score),
                                      _stream(stream))
    _check(st, "nsa_update_block_reps")


def nsa_select_workspace_bytes(shape: Shape, params: SelectParams, max_seq_len: int) -> int:
    out = ctypes.c_size_t(0)
    st = load().nsa_select_workspace_bytes(ctypes.byref(shape), ctypes.byref(params),
                                           int(max_seq_len), ctypes.byref(out))
    _check(st, "nsa_select_workspace_bytes")
    return out.value


def nsa_select_blocks(shape: Shape, params: SelectParams, query, reps, evict_block_score,
                      seq_lens, max_seq_len: int, evict_set, evict_seen, selected, num_selected,
                      workspace, workspace_bytes: int, stream=None) -> None:
    st = load().nsa_select_blocks(ctypes.byref(shape), ctypes.byref(params), _ptr(query),
                                  _ptr(reps), _ptr(evict_block_score), _ptr(seq_lens),
                                  int(max_seq_len), _ptr(evict_set), _ptr(evict_seen),
                                  _ptr(selected), _ptr(num_selected), _ptr(workspace),
                                  int(workspace_bytes), _stream(stream))
    _check(st, "nsa_select_blocks")


def nsa_decode_workspace_bytes(shape: Shape, params: DecodeParams) -> int:
    out = ctypes.c_size_t(0)
    st = load().nsa_decode_workspace_bytes(ctypes.byref(shape), ctypes.byref(params),
                                           ctypes.byref(out))
    _check(st, "nsa_decode_workspace_bytes")
    return out.value


def nsa_sparse_decode(shape: Shape, params: DecodeParams, q, k_pool, v_pool, block_table,
                      seq_lens, selected, num_selected, num_processed, out, workspace,
                      workspace_bytes: int, stream=None) -> None:
    st = load().nsa_sparse_decode(ctypes.byref(shape), ctypes.byref(params), _ptr(q),
                                  _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens),
                                  _ptr(selected), _ptr(num_selected), _ptr(num_processed),
                                  _ptr(out), _ptr(workspace), int(workspace_bytes),
                                  _stream(stream))
    _check(st, "nsa_sparse_decode")


def nsa_sparse_decode_biased(shape: Shape, params: DecodeParams, q, k_pool, v_pool, block_table,
                             seq_lens, selected, num_selected, attn_bias, num_processed, out,
                             workspace, workspace_bytes: int, stream=None) -> None:
    st = load().nsa_sparse_decode_biased(ctypes.byref(shape), ctypes.byref(params), _ptr(q),
                                         _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                         _ptr(seq_lens), _ptr(selected), _ptr(num_selected),
                                         _ptr(attn_bias), _ptr(num_processed), _ptr(out),
                                         _ptr(workspace), int(workspace_bytes), _stream(stream))
    _check(st, "nsa_sparse_decode_biased")


def nsa_decode_step_workspace_bytes(shape: Shape, params: SelectParams, max_seq_len: int) -> int:
    out = ctypes.c_size_t(0)
    st = load().nsa_decode_step_workspace_bytes(ctypes.byref(shape), ctypes.byref(params),
                                                int(max_seq_len), ctypes.byref(out))
    _check(st, "nsa_decode_step_workspace_bytes")
    return out.value


def nsa_decode_step(shape: Shape, params: SelectParams, query, q, reps, evict_block_score,
                    k_pool, v_pool, block_table, seq_lens, max_seq_len: int, evict_set,
                    evict_seen, selected, num_selected, out, workspace, workspace_bytes: int,
                    stream=None) -> None:
    st = load().nsa_decode_step(ctypes.byref(shape), ctypes.byref(params), _ptr(query), _ptr(q),
                                _ptr(reps), _ptr(evict_block_score), _ptr(k_pool), _ptr(v_pool),
                                _ptr(block_table), _ptr(seq_lens), int(max_seq_len),
                                _ptr(evict_set), _ptr(evict_seen), _ptr(selected),
                                _ptr(num_selected), _ptr(out), _ptr(workspace),
                                int(workspace_bytes), _stream(stream))
    _check(st, "nsa_decode_step")


def nsa_decode_step_status(workspace, workspace_bytes: int, clear: bool = True,
                           stream=None) -> None:
    """Raises NsaError(NSA_ERR_STEP_EXPIRED) when a wait of a fused step run on
    this workspace expired (synchronises the stream)."""
    st = load().nsa_decode_step_status(_ptr(workspace), int(workspace_bytes), int(bool(clear)),
                                       _stream(stream))
    _check(st, "nsa_decode_step_status")


def nsa_residency_diff(shape: Shape, max_selected: int, prev_selected, prev_num_selected,
                       prev_seq_lens, selected, num_selected, fetch, num_fetch, release,
                       num_release, gamma=None, stream=None) -> None:
    st = load().nsa_residency_diff(ctypes.byref(shape), int(max_selected), _ptr(prev_selected),
                                   _ptr(prev_num_selected), _ptr(prev_seq_lens), _ptr(selected),
                                   _ptr(num_selected), _ptr(fetch), _ptr(num_fetch),
                                   _ptr(release), _ptr(num_release), _ptr(gamma),
                                   _stream(stream))
    _check(st, "nsa_residency_diff")


def nsa_s2o_workspace_bytes(shape: Shape, params: PrefillParams) -> int:
    out = ctypes.c_size_t(0)
    st = load().nsa_s2o_workspace_bytes(ctypes.byref(shape), ctypes.byref(params),
                                        ctypes.byref(out))
    _check(st, "nsa_s2o_workspace_bytes")
    return out.value


def nsa_s2o_index(shape: Shape, params: PrefillParams, q, k_pool, block_table, seq_lens, q_perm,
                  kv_perm, workspace, workspace_bytes: int, stream=None) -> None:
    st = load().nsa_s2o_index(ctypes.byref(shape), ctypes.byref(params), _ptr(q), _ptr(k_pool),
                              _ptr(block_table), _ptr(seq_lens), _ptr(q_perm), _ptr(kv_perm),
                              _ptr(workspace), int(workspace_bytes), _stream(stream))
    _check(st, "nsa_s2o_index")


def nsa_s2o_attend(shape: Shape, params: PrefillParams, q, k_pool, v_pool, block_table, seq_lens,
                   q_perm, kv_perm, out, num_tiles, workspace, workspace_bytes: int,
                   stream=None) -> None:
    st = load().nsa_s2o_attend(ctypes.byref(shape), ctypes.byref(params), _ptr(q), _ptr(k_pool),
                               _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), _ptr(q_perm),
                               _ptr(kv_perm), _ptr(out), _ptr(num_tiles), _ptr(workspace),
                               int(workspace_bytes), _stream(stream))
    _check(st, "nsa_s2o_attend")


def nsa_decode_step_noalloc(shape: Shape, params: SelectParams, query, q, reps, evict_block_score,
                            k_pool, v_pool, block_table, seq_lens, max_seq_len: int, evict_set,
                            evict_seen, selected, num_selected, out, step_status=None,
                            stream=None) -> None:
    st = load().nsa_decode_step_noalloc(ctypes.byref(shape), ctypes.byref(params), _ptr(query),
                                        _ptr(q), _ptr(reps), _ptr(evict_block_score),
                                        _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                        _ptr(seq_lens), int(max_seq_len), _ptr(evict_set),
                                        _ptr(evict_seen), _ptr(selected), _ptr(num_selected),
                                        _ptr(out), _ptr(step_status), _stream(stream))
    _check(st, "nsa_decode_step_noalloc")


def nsa_debug_checks() -> bool:
    return bool(load().nsa_debug_checks())


def nsa_debug_error(clear: bool = True) -> int:
    """The OR of the device-side contract violations recorded since the last
    clear (0 unless the library was built with the checks)."""
    out = ctypes.c_uint32(0)
    st = load().nsa_debug_error(ctypes.byref(out), int(bool(clear)))
    _check(st, "nsa_debug_error")
    return out.value


def nsa_decode_step_grid(shape: Shape, params: SelectParams, max_seq_len: int,
                         capacity: int) -> StepGrid:
    out = StepGrid()
    st = load().nsa_decode_step_grid(ctypes.byref(shape), ctypes.byref(params), int(max_seq_len),
                                     int(capacity), ctypes.byref(out))
    _check(st, "nsa_decode_step_grid")
    return out
