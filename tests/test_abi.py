"""CPU checks of the C ABI: the library loads, exports every function that
include/nsa.h declares, and rejects bad arguments before any HIP call (no
kernel is launched here)."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nsa.h")

N = pytest.importorskip("block_sparse_kv_nsa_amd")

FAKE = 1 << 20            # non-NULL, 256-aligned stand-in pointer (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:nsa_status|const char\*|int32_t)\s+(nsa_\w+)\s*\(",
                                 text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    lib = N.load()
    names = declared_functions()
    assert len(names) == 20, names
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(N.EXPORTS) == names


def test_abi_version_matches_header():
    m = re.search(r"#define NSA_ABI_VERSION (\d+)", open(HEADER).read())
    assert N.nsa_abi_version() == int(m.group(1))


def test_status_strings():
    assert N.nsa_status_string(0) == "NSA_OK"
    assert N.nsa_status_string(3) == "NSA_ERR_WORKSPACE_TOO_SMALL"
    assert N.nsa_status_string(99) == "NSA_ERR_UNKNOWN"


def shape(**kw):
    base = dict(batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128, max_blocks_per_seq=2049,
                num_phys_blocks=8196, dtype=N.NSA_BF16)
    base.update(kw)
    return N.Shape.make(**base)


def expect(status, fn, *args):
    with pytest.raises(N.NsaError) as ei:
        fn(*args)
    assert ei.value.status == status, str(ei.value)
    return str(ei.value)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), N.NSA_ERR_UNSUPPORTED),
    (dict(num_q_heads=24), N.NSA_ERR_UNSUPPORTED),          # group 3
    (dict(num_q_heads=30), N.NSA_ERR_INVALID_ARGUMENT),     # not a multiple
    (dict(batch=0), N.NSA_ERR_INVALID_ARGUMENT),
    (dict(max_blocks_per_seq=20000), N.NSA_ERR_INVALID_ARGUMENT),
    (dict(dtype=7), N.NSA_ERR_INVALID_ARGUMENT),
    (dict(block_size=32), N.NSA_ERR_UNSUPPORTED),
    (dict(sub_block=8), N.NSA_ERR_UNSUPPORTED),
])
def test_shape_validation(kw, status):
    expect(status, N.nsa_decode_workspace_bytes, shape(**kw), N.DecodeParams(64, 0, 0.0))


@pytest.mark.parametrize("params,status", [
    (N.SelectParams(0, 64, 65, 0), N.NSA_ERR_INVALID_ARGUMENT),   # k_e > k
    (N.SelectParams(0, 0, 0, 0), N.NSA_ERR_INVALID_ARGUMENT),     # k = 0
    (N.SelectParams(3, 64, 0, 0), N.NSA_ERR_INVALID_ARGUMENT),    # mode
    (N.SelectParams(0, 64, 8, 1), N.NSA_ERR_INVALID_ARGUMENT),    # ordered with k_e
    (N.SelectParams(0, 5000, 0, 0), N.NSA_ERR_INVALID_ARGUMENT),  # k too large
])
def test_select_param_validation(params, status):
    expect(status, N.nsa_select_workspace_bytes, shape(), params, 131088)


def test_select_workspace_grows_with_context():
    p = N.SelectParams(0, 64, 48, 0)
    a = N.nsa_select_workspace_bytes(shape(), p, 4096)
    b = N.nsa_select_workspace_bytes(shape(), p, 131088)
    assert 0 < a < b
    expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_select_workspace_bytes, shape(), p, 64 * 2049 + 1)


def test_null_and_alignment_rejected_before_launch():
    s, p = shape(), N.SelectParams(0, 64, 48, 0)
    ws = N.nsa_select_workspace_bytes(s, p, 131088)
    args = [s, p, FAKE, FAKE, FAKE, FAKE, 131088, FAKE, FAKE, FAKE, FAKE, FAKE, ws, 0]
    for i, name in ((2, "query"), (3, "reps"), (5, "seq_lens"), (9, "selected"), (11, "workspace")):
        bad = list(args)
        bad[i] = None
        msg = expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_select_blocks, *bad)
        assert name in msg
    bad = list(args)
    bad[2] = FAKE + 2                  # query not 16-byte aligned
    expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_select_blocks, *bad)
    bad = list(args)
    bad[4] = None                      # E required when k_e > 0
    expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_select_blocks, *bad)
    small = list(args)
    small[12] = ws - 256
    expect(N.NSA_ERR_WORKSPACE_TOO_SMALL, N.nsa_select_blocks, *small)
    assert "workspace" in N.nsa_last_error()


def test_decode_validation():
    s = shape()
    d = N.DecodeParams(64, 1, 1e-3)
    ws = N.nsa_decode_workspace_bytes(s, d)
    args = [s, d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, 0]
    bad = list(args)
    bad[9] = None                      # num_processed needed for early stop
    expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_sparse_decode, *bad)
    expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_decode_workspace_bytes, s, N.DecodeParams(64, 0, -1.0))
    expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_decode_workspace_bytes, s, N.DecodeParams(0, 0, 0.0))
    small = list(args)
    small[12] = 0
    expect(N.NSA_ERR_WORKSPACE_TOO_SMALL, N.nsa_sparse_decode, *small)
    # the biased form: the bias after num_selected, required and 4-byte aligned
    biased = args[:9] + [FAKE] + args[9:]
    nobias = list(biased)
    nobias[9] = None
    expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_sparse_decode_biased, *nobias)
    odd = list(biased)
    odd[9] = FAKE + 2
    expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_sparse_decode_biased, *odd)
    small = list(biased)
    small[13] = 0
    expect(N.NSA_ERR_WORKSPACE_TOO_SMALL, N.nsa_sparse_decode_biased, *small)


def test_reps_validation_and_noop():
    s = shape()
    expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_update_block_reps, s, FAKE, FAKE, FAKE, FAKE, FAKE,
           1, FAKE, None)                                 # logits without scores
    expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_update_block_reps, s, FAKE, FAKE, None, FAKE, FAKE,
           5000, FAKE, None)                              # more blocks than capacity
    N.nsa_update_block_reps(s, FAKE, FAKE, None, FAKE, FAKE, 0, FAKE, None)   # nothing to do


def test_product_path_has_no_fallback():
    """The package refuses to import without the built library."""
    import importlib
    import subprocess
    import sys
    code = ("import os, block_sparse_kv_nsa_amd._abi as A; A.LIB_PATH = '/nonexistent/libnsa.so'; "
            "A._lib = None\ntry:\n    A.load()\nexcept ImportError:\n    print('raised')")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert "raised" in r.stdout, r.stderr


def test_step_status_validation():
    """The status query checks its arguments before any HIP call."""
    expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_decode_step_status, None, 4096)
    expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_decode_step_status, FAKE + 16, 4096)
    expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_decode_step_status, FAKE, 128)
    assert N.nsa_status_string(N.NSA_ERR_STEP_EXPIRED) == "NSA_ERR_STEP_EXPIRED"


def test_residency_diff_validation():
    s = shape()
    args = [s, 64] + [FAKE] * 9 + [None, 0]
    for i in range(2, 11):
        bad = list(args)
        bad[i] = None
        expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_residency_diff, *bad)
    bad = list(args)
    bad[1] = 0
    expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_residency_diff, *bad)
    bad = list(args)
    bad[11] = FAKE + 2                 # gamma misaligned
    expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_residency_diff, *bad)


def test_step_noalloc_validation():
    """Arguments and the per-device size limit are checked before any HIP call."""
    s, p = shape(), N.SelectParams(0, 64, 48, 0)
    args = [s, p] + [FAKE] * 8 + [131088] + [FAKE] * 5 + [None, 0]
    bad = list(args)
    bad[2] = None
    expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_decode_step_noalloc, *bad)
    bad = list(args)
    bad[16] = FAKE + 2                 # status misaligned
    expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_decode_step_noalloc, *bad)
    big = list(args)                   # 512 rows x 8 heads of head_dim 128: above the limit
    big[0] = shape(batch=256, num_q_heads=64, num_kv_heads=8)
    msg = expect(N.NSA_ERR_UNSUPPORTED, N.nsa_decode_step_noalloc, *big)
    assert "per device" in msg
    ordered = list(args)
    ordered[1] = N.SelectParams(0, 64, 0, 1)
    expect(N.NSA_ERR_UNSUPPORTED, N.nsa_decode_step_noalloc, *ordered)


def test_debug_checks_queries():
    """Release builds report no checks and an empty error word, without any
    device call; a NULL output is rejected."""
    lib = N.load()
    if N.nsa_debug_checks():
        pytest.skip("a build with the device checks")
    assert N.nsa_debug_error() == 0
    assert lib.nsa_debug_error(None, 0) == N.NSA_ERR_INVALID_ARGUMENT


def test_s2o_validation():
    """S2O prefill arguments are checked before any HIP call."""
    sh = shape(batch=1, max_blocks_per_seq=512, num_phys_blocks=512)
    ok = N.PrefillParams(1024, 32768, 1e-3)
    ptrs = [FAKE] * 7
    expect(N.NSA_ERR_UNSUPPORTED, N.nsa_s2o_workspace_bytes, shape(dtype=N.NSA_F32), ok)
    for bad in (N.PrefillParams(96, 32768, 1e-3), N.PrefillParams(8192, 32768, 1e-3),
                N.PrefillParams(1024, 32768 + 32, 1e-3), N.PrefillParams(1024, 64 * 513, 1e-3),
                N.PrefillParams(1024, 32768, -1.0), N.PrefillParams(1024, 32768, float("inf"))):
        expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_s2o_workspace_bytes, sh, bad)
        expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_s2o_index, sh, bad, *ptrs, 1 << 30)
        expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_s2o_attend, sh, bad, *ptrs, FAKE, FAKE, FAKE,
               1 << 30)
    big = shape(batch=64, max_blocks_per_seq=2048, num_phys_blocks=2048 * 64)
    expect(N.NSA_ERR_UNSUPPORTED, N.nsa_s2o_workspace_bytes, big, N.PrefillParams(1024, 131072, 0))
    msg = expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_s2o_attend, sh, ok, FAKE, FAKE, FAKE, FAKE,
                 FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 40)
    assert "out" in msg
    msg = expect(N.NSA_ERR_WORKSPACE_TOO_SMALL, N.nsa_s2o_attend, sh, ok, FAKE, FAKE, FAKE, FAKE,
                 FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096)
    assert "workspace" in msg
    msg = expect(N.NSA_ERR_INVALID_ARGUMENT, N.nsa_s2o_index, sh, ok, FAKE + 2, FAKE, FAKE, FAKE,
                 FAKE, FAKE, FAKE, 1 << 30)
    assert "aligned" in msg
