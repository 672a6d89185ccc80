"""The C-ABI library loads on the host and exports what include/sgemm.h declares.

These tests make no compute call: they need no GPU.  Host-only behaviour
(status names, argument checks that precede any runtime call) is exercised
through the same ctypes binding the GPU tests use.
"""
import ctypes
import os
import re

import pytest

import dense_fp32_matrix_03_amd as sg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^[\w\s\*]*?\b(\w+)\s*\([^;{]*\)\s*;", text, flags=re.M)
    return names


def test_header_declares_the_entry_points():
    names = set(_declared_functions())
    for n in ("sgemm_create", "sgemm_run", "sgemm_destroy", "sgemm_run_variant",
              "sgemm_run_ex", "sgemm_run_strided_batched", "vector_add", "sgemm_mfma_probe",
              "sgemm_bf16x3_workspace_size", "sgemm_run_bf16x3", "sgemm_run_bf16x3_ex",
              "sgemm_mfma_ceiling", "sgemm_status_string", "sgemm_variant_name",
              "sgemm_phase_times", "sgemm_run_bf16x3_ex_noalloc"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(sg.LIB_PATH)
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings():
    for name, code in sg._C.items():
        if name.startswith("SGEMM_ERR_") or name == "SGEMM_OK":
            assert sg.sgemm_status_string(code) == name
    assert sg.sgemm_status_string(12345) == "unknown status"


def test_variant_names():
    for key, v in sg.VARIANTS.items():
        assert sg.sgemm_variant_name(v) is not None
    assert sg.sgemm_variant_name(sg.NUM_VARIANTS) is None
    assert sg.sgemm_variant_name(-1) is None


@pytest.mark.parametrize("args,status", [
    ((-1, 4, 4, 1, 4, 1, 4, 1, 4), "SGEMM_ERR_INVALID_VALUE"),   # negative M
    ((4, 4, 4, 1, 3, 1, 4, 1, 4), "SGEMM_ERR_INVALID_VALUE"),    # lda < K
    ((4, 4, 4, 1, 4, 1, 3, 1, 4), "SGEMM_ERR_INVALID_VALUE"),    # ldb < N
    ((4, 4, 4, 1, 4, 1, 4, 1, 3), "SGEMM_ERR_INVALID_VALUE"),    # ldc < N
    ((4, 4, 4, 0, 4, 1, 4, 1, 4), "SGEMM_ERR_INVALID_VALUE"),    # null A
    ((4, 4, 4, 1, 4, 1, 4, 0, 4), "SGEMM_ERR_INVALID_VALUE"),    # null C
    ((2 ** 31, 4, 4, 1, 4, 1, 4, 1, 4), "SGEMM_ERR_TOO_LARGE"),
    ((4, 4, 4, 1, 4, 1, 4, 1, 4), "SGEMM_ERR_NOT_INITIALIZED"),  # valid, before create
])
def test_host_side_argument_checks(args, status):
    lib = sg.load_library()
    M, N, K, A, lda, B, ldb, C, ldc = args
    rc = lib.sgemm_run(M, N, K, A or None, lda, B or None, ldb, C or None, ldc, None)
    assert sg.sgemm_status_string(rc) == status
    rc = lib.sgemm_run_variant(0, M, N, K, A or None, lda, B or None, ldb, C or None, ldc, None)
    assert sg.sgemm_status_string(rc) == status


def test_unknown_variant_rejected():
    lib = sg.load_library()
    rc = lib.sgemm_run_variant(sg.NUM_VARIANTS, 4, 4, 4, 1, 4, 1, 4, 1, 4, None)
    assert sg.sgemm_status_string(rc) == "SGEMM_ERR_INVALID_VALUE"
    rc = lib.sgemm_mfma_probe(3, 1, 1, 1, None)
    assert sg.sgemm_status_string(rc) == "SGEMM_ERR_INVALID_VALUE"


def test_forced_tile_work_item_limits():
    """A launch must stay below 2^32 work-items.  At 200000 x 200000 the
    64 x 64 blocks number 3125^2: sgemm_run takes the product (it picks a
    tile whose launch fits), but the forced 64 x 64 tile (512 per block),
    32 x 64 and 32 x 32 tiles (256 per block) would not fit; at 131072^2 the
    forced 64 x 64 tile does.  The checks come before anything touches the
    runtime."""
    lib = sg.load_library()

    def status(variant, n):
        return sg.sgemm_status_string(
            lib.sgemm_run_variant(sg.VARIANTS[variant], n, n, 1, 16, 1, 16, n, 16, n, None))

    for v in ("mfma_64", "mfma_32x64", "mfma_32", "dbuf"):
        assert status(v, 200000) == "SGEMM_ERR_TOO_LARGE", v
    for v in ("mfma", "mfma_128", "mfma_256"):
        assert status(v, 200000) == "SGEMM_ERR_NOT_INITIALIZED", v
    assert status("mfma_64", 131072) == "SGEMM_ERR_NOT_INITIALIZED"


def test_destroy_without_create():
    lib = sg.load_library()
    assert sg.sgemm_status_string(lib.sgemm_destroy()) == "SGEMM_ERR_NOT_INITIALIZED"


# (transA, transB, M, N, K, lda, ldb, ldc, strideA, strideB, strideC, batch), status
@pytest.mark.parametrize("args,status", [
    ((2, 0, 4, 4, 4, 4, 4, 4, 0, 0, 16, 1), "SGEMM_ERR_INVALID_VALUE"),   # bad transA
    ((0, -1, 4, 4, 4, 4, 4, 4, 0, 0, 16, 1), "SGEMM_ERR_INVALID_VALUE"),  # bad transB
    ((1, 0, 8, 4, 4, 4, 4, 4, 0, 0, 32, 1), "SGEMM_ERR_INVALID_VALUE"),   # transA: lda < M
    ((0, 1, 4, 8, 6, 6, 4, 8, 0, 0, 32, 1), "SGEMM_ERR_INVALID_VALUE"),   # transB: ldb < K
    ((0, 1, 4, 8, 6, 6, 6, 8, 0, 0, 32, 1), "SGEMM_ERR_NOT_INITIALIZED"),  # transB: ldb >= K
    ((0, 0, 4, 4, 4, 4, 4, 4, -4, 0, 16, 2), "SGEMM_ERR_INVALID_VALUE"),  # negative stride
    ((0, 0, 4, 4, 4, 4, 4, 4, 0, 0, 15, 2), "SGEMM_ERR_INVALID_VALUE"),   # C matrices overlap
    ((0, 0, 4, 4, 4, 4, 4, 8, 0, 0, 28, 2), "SGEMM_ERR_NOT_INITIALIZED"),  # (M-1)ldc+N = 28
    ((0, 0, 4, 4, 4, 4, 4, 4, 0, 0, 0, 1), "SGEMM_ERR_NOT_INITIALIZED"),  # one product
    ((0, 0, 4, 4, 4, 4, 4, 4, 0, 0, 16, -1), "SGEMM_ERR_INVALID_VALUE"),  # negative batch
    ((0, 0, 4, 4, 4, 4, 4, 4, 0, 0, 16, 2 ** 31), "SGEMM_ERR_TOO_LARGE"),
    # one 256-thread work-group per product: 2^24 of them is 2^32 work-items
    ((0, 0, 64, 64, 4, 4, 64, 64, 0, 0, 4096, 2 ** 24 - 1), "SGEMM_ERR_NOT_INITIALIZED"),
    ((0, 0, 64, 64, 4, 4, 64, 64, 0, 0, 4096, 2 ** 24), "SGEMM_ERR_TOO_LARGE"),
])
def test_general_host_side_argument_checks(args, status):
    lib = sg.load_library()
    ta, tb, M, N, K, lda, ldb, ldc, sA, sB, sC, batch = args
    rc = lib.sgemm_run_strided_batched(ta, tb, M, N, K, 1.0, 1, lda, sA, 1, ldb, sB, 0.0, 1, ldc,
                                       sC, batch, None)
    assert sg.sgemm_status_string(rc) == status
    if batch == 1:
        rc = lib.sgemm_run_ex(ta, tb, M, N, K, 1.0, 1, lda, 1, ldb, 0.0, 1, ldc, None)
        assert sg.sgemm_status_string(rc) == status


def test_general_null_operands():
    lib = sg.load_library()
    # alpha == 0: A and B are not read, so they may be NULL
    rc = lib.sgemm_run_ex(0, 0, 4, 4, 4, 0.0, None, 4, None, 4, 1.0, 1, 4, None)
    assert sg.sgemm_status_string(rc) == "SGEMM_ERR_NOT_INITIALIZED"
    rc = lib.sgemm_run_ex(0, 0, 4, 4, 4, 1.0, None, 4, 1, 4, 1.0, 1, 4, None)
    assert sg.sgemm_status_string(rc) == "SGEMM_ERR_INVALID_VALUE"
    rc = lib.sgemm_run_ex(0, 0, 4, 4, 4, 1.0, 1, 4, 1, 4, 1.0, None, 4, None)
    assert sg.sgemm_status_string(rc) == "SGEMM_ERR_INVALID_VALUE"


@pytest.mark.parametrize("n,ptr,status", [
    (-1, 1, "SGEMM_ERR_INVALID_VALUE"),
    (4, 0, "SGEMM_ERR_INVALID_VALUE"),
    (2 ** 33 + 1, 1, "SGEMM_ERR_TOO_LARGE"),
    (2 ** 33, 1, "SGEMM_ERR_NOT_INITIALIZED"),
    (4, 1, "SGEMM_ERR_NOT_INITIALIZED"),
    (0, 0, "SGEMM_ERR_NOT_INITIALIZED"),
])
def test_vector_add_host_side_argument_checks(n, ptr, status):
    lib = sg.load_library()
    rc = lib.vector_add(n, 1, ptr or None, 1, None)
    assert sg.sgemm_status_string(rc) == status


def test_bf16x3_workspace_size_and_host_checks():
    lib = sg.load_library()
    assert lib.sgemm_bf16x3_workspace_size(100, 50, 33) == 6 * 64 * 150
    assert lib.sgemm_bf16x3_workspace_size(100, 50, 0) == 0
    assert sg.sgemm_status_string(lib.sgemm_bf16x3_workspace_size(-1, 5, 5)) == \
        "SGEMM_ERR_INVALID_VALUE"
    assert sg.sgemm_status_string(lib.sgemm_bf16x3_workspace_size(5, 5, 2 ** 21 + 1)) == \
        "SGEMM_ERR_TOO_LARGE"
    assert sg.sgemm_status_string(lib.sgemm_bf16x3_workspace_size(2 ** 30, 2 ** 30, 64)) == \
        "SGEMM_ERR_TOO_LARGE"
    need = lib.sgemm_bf16x3_workspace_size(4, 4, 4)
    run = lib.sgemm_run_bf16x3
    assert sg.sgemm_status_string(run(4, 4, 4, 16, 4, 16, 4, 16, 4, 256, need, None)) == \
        "SGEMM_ERR_NOT_INITIALIZED"
    assert sg.sgemm_status_string(run(4, 4, 4, 16, 4, 16, 4, 16, 4, 256, need - 1, None)) == \
        "SGEMM_ERR_INVALID_VALUE"
    assert sg.sgemm_status_string(run(4, 4, 4, 16, 4, 16, 4, 16, 4, 264, need, None)) == \
        "SGEMM_ERR_INVALID_VALUE"
    assert sg.sgemm_status_string(run(4, 4, 4, 16, 4, 16, 4, 16, 4, None, need, None)) == \
        "SGEMM_ERR_INVALID_VALUE"
    assert sg.sgemm_status_string(run(4, 4, 4, 16, 3, 16, 4, 16, 4, 256, need, None)) == \
        "SGEMM_ERR_INVALID_VALUE"


def test_bf16x3_ex_host_checks():
    lib = sg.load_library()
    ex = lib.sgemm_run_bf16x3_ex

    def st(*args):
        return sg.sgemm_status_string(ex(*args))

    # (transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, ws, ws_bytes, stream)
    M, N, K = 6, 5, 3
    need = lib.sgemm_bf16x3_workspace_size(M, N, K)
    assert st(0, 0, M, N, K, 1, 16, K, 16, N, 0, 16, N, 256, need, None) == \
        "SGEMM_ERR_NOT_INITIALIZED"
    assert st(2, 0, M, N, K, 1, 16, K, 16, N, 0, 16, N, 256, need, None) == \
        "SGEMM_ERR_INVALID_VALUE"
    assert st(0, -1, M, N, K, 1, 16, K, 16, N, 0, 16, N, 256, need, None) == \
        "SGEMM_ERR_INVALID_VALUE"
    # Leading dimensions follow the stored shapes: A^T is K x M, B^T is N x K.
    assert st(1, 0, M, N, K, 1, 16, K, 16, N, 0, 16, N, 256, need, None) == \
        "SGEMM_ERR_INVALID_VALUE"
    assert st(1, 0, M, N, K, 1, 16, M, 16, N, 0, 16, N, 256, need, None) == \
        "SGEMM_ERR_NOT_INITIALIZED"
    assert st(0, 1, M, N, K, 1, 16, K, 16, K - 1, 0, 16, N, 256, need, None) == \
        "SGEMM_ERR_INVALID_VALUE"
    assert st(0, 1, M, N, K, 1, 16, K, 16, K, 0, 16, N, 256, need, None) == \
        "SGEMM_ERR_NOT_INITIALIZED"
    assert st(0, 0, M, N, K, 1, 16, K, 16, N, 0, 16, N - 1, 256, need, None) == \
        "SGEMM_ERR_INVALID_VALUE"
    # The workspace is checked only when the product is formed.
    assert st(0, 0, M, N, K, 1, 16, K, 16, N, 0, 16, N, 256, need - 1, None) == \
        "SGEMM_ERR_INVALID_VALUE"
    assert st(0, 0, M, N, K, 1, 16, K, 16, N, 0, 16, N, 264, need, None) == \
        "SGEMM_ERR_INVALID_VALUE"
    assert st(0, 0, M, N, K, 0, None, K, None, N, 2, 16, N, None, 0, None) == \
        "SGEMM_ERR_NOT_INITIALIZED"
    assert st(0, 0, M, N, 0, 1, None, 1, None, N, 2, 16, N, None, 0, None) == \
        "SGEMM_ERR_NOT_INITIALIZED"
    assert st(0, 0, M, N, K, 1, None, K, 16, N, 0, 16, N, 256, need, None) == \
        "SGEMM_ERR_INVALID_VALUE"
    assert st(0, 0, M, N, K, 1, 16, K, 16, N, 0, None, N, 256, need, None) == \
        "SGEMM_ERR_INVALID_VALUE"
    # Size limits of the split apply only when the product is formed.
    assert st(0, 0, M, N, 2 ** 21 + 1, 1, 16, 2 ** 21 + 1, 16, N, 0, 16, N, 256, 1 << 40,
              None) == "SGEMM_ERR_TOO_LARGE"
    assert st(0, 0, M, N, 2 ** 21 + 1, 0, 16, 2 ** 21 + 1, 16, N, 0, 16, N, None, 0,
              None) == "SGEMM_ERR_NOT_INITIALIZED"


def test_mfma_ceiling_host_checks():
    lib = sg.load_library()
    f = ctypes.c_double()
    for which, iters, out in ((2, 10, 16), (0, 0, 16), (0, 10, 0)):
        rc = lib.sgemm_mfma_ceiling(which, iters, out or None, 1 << 20, ctypes.byref(f), None)
        assert sg.sgemm_status_string(rc) == "SGEMM_ERR_INVALID_VALUE"
    rc = lib.sgemm_mfma_ceiling(0, 10, 16, 1 << 20, ctypes.byref(f), None)
    assert sg.sgemm_status_string(rc) == "SGEMM_ERR_NOT_INITIALIZED"
