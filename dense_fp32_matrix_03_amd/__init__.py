"""Python binding of libsgemm: single-precision C = A x B on MI355X (gfx950).

Argument marshalling only.  Every function here forwards to the entry point
of the same name in libsgemm.so (declared in include/sgemm.h); all arithmetic
runs in the library's HIP kernels.  There is no CPU fallback: if the library
is missing, every call raises.

Matrices may be given as torch tensors on the GPU (their data pointer is
passed) or as plain integer device addresses.  ``stream`` may be a
torch.cuda.Stream, an integer hipStream_t, or None for torch's current stream
on the current device.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsgemm.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "sgemm.h")


def _header_constants() -> dict:
    out = {}
    with open(HEADER_PATH) as f:
        for m in re.finditer(r"#define\s+(SGEMM_\w+)\s+\(?(-?\d+)\)?", f.read()):
            out[m.group(1)] = int(m.group(2))
    return out


_C = _header_constants()
SGEMM_OK = _C["SGEMM_OK"]
VARIANTS = {k[len("SGEMM_VARIANT_"):].lower(): v for k, v in _C.items()
            if k.startswith("SGEMM_VARIANT_")}
NUM_VARIANTS = _C["SGEMM_NUM_VARIANTS"]


class SgemmError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {sgemm_status_string(status)} ({status})")


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libsgemm.so and declare its signatures (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python -m dense_fp32_matrix_03_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    gemm_args = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp]
    lib.sgemm_create.argtypes = []
    lib.sgemm_create.restype = ci
    lib.sgemm_destroy.argtypes = []
    lib.sgemm_destroy.restype = ci
    lib.sgemm_run.argtypes = gemm_args
    lib.sgemm_run.restype = ci
    lib.sgemm_run_variant.argtypes = [ci] + gemm_args
    lib.sgemm_run_variant.restype = ci
    f32 = ctypes.c_float
    lib.sgemm_run_ex.argtypes = [ci, ci, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, vp]
    lib.sgemm_run_ex.restype = ci
    lib.sgemm_run_strided_batched.argtypes = [ci, ci, i64, i64, i64, f32, vp, i64, i64, vp, i64,
                                              i64, f32, vp, i64, i64, i64, vp]
    lib.sgemm_run_strided_batched.restype = ci
    lib.sgemm_bf16x3_workspace_size.argtypes = [i64, i64, i64]
    lib.sgemm_bf16x3_workspace_size.restype = i64
    lib.sgemm_run_bf16x3.argtypes = gemm_args[:-1] + [vp, i64, vp]
    lib.sgemm_run_bf16x3.restype = ci
    lib.sgemm_run_bf16x3_ex.argtypes = [ci, ci, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp,
                                        i64, vp, i64, vp]
    lib.sgemm_run_bf16x3_ex.restype = ci
    lib.sgemm_run_bf16x3_ex_noalloc.argtypes = [ci, ci, i64, i64, i64, f32, vp, i64, vp, i64,
                                                f32, vp, i64, vp]
    lib.sgemm_run_bf16x3_ex_noalloc.restype = ci
    lib.vector_add.argtypes = [i64, vp, vp, vp, vp]
    lib.vector_add.restype = ci
    lib.sgemm_mfma_ceiling.argtypes = [ci, ci, vp, i64, ctypes.POINTER(ctypes.c_double), vp]
    lib.sgemm_mfma_ceiling.restype = ci
    lib.sgemm_phase_times.argtypes = gemm_args[:-1] + [vp, i64, ctypes.POINTER(i64), vp]
    lib.sgemm_phase_times.restype = ci
    pi = ctypes.POINTER(ci)
    lib.sgemm_tile_choice.argtypes = [i64, i64, i64, i64, ci, pi, pi, pi, pi]
    lib.sgemm_tile_choice.restype = ci
    lib.sgemm_mfma_probe.argtypes = [ci, vp, vp, vp, vp]
    lib.sgemm_mfma_probe.restype = ci
    lib.sgemm_status_string.argtypes = [ci]
    lib.sgemm_status_string.restype = ctypes.c_char_p
    lib.sgemm_variant_name.argtypes = [ci]
    lib.sgemm_variant_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if getattr(x, "device", None) is not None and x.device.type != "cuda":
            raise ValueError("tensor must live on the GPU")
        return x.data_ptr()
    raise TypeError(f"cannot take a device pointer from {type(x).__name__}")


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(fn: str, status: int) -> None:
    if status != SGEMM_OK:
        raise SgemmError(fn, status)


def sgemm_create() -> None:
    _check("sgemm_create", load_library().sgemm_create())


def sgemm_destroy() -> None:
    _check("sgemm_destroy", load_library().sgemm_destroy())


def sgemm_run(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> None:
    """C = A x B (row-major, leading dimensions lda, ldb, ldc) on `stream`."""
    _check("sgemm_run", load_library().sgemm_run(
        M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _stream(stream)))


def sgemm_run_variant(variant, M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> None:
    """sgemm_run computed by kernel `variant` (an int or a VARIANTS key)."""
    v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    _check("sgemm_run_variant", load_library().sgemm_run_variant(
        v, M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _stream(stream)))


def sgemm_run_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                 stream=None) -> None:
    """C = alpha op(A) op(B) + beta C (op = transpose when the flag is set)."""
    _check("sgemm_run_ex", load_library().sgemm_run_ex(
        int(transA), int(transB), M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb,
        float(beta), _ptr(C), ldc, _stream(stream)))


def sgemm_tile_choice(M, N, K, batch=1, cus=256) -> tuple:
    """(bm, bn, bk, ksets) that sgemm_run and the general form choose for
    `batch` products of M x N x K on `cus` compute units (host logic only)."""
    out = [ctypes.c_int() for _ in range(4)]
    _check("sgemm_tile_choice", load_library().sgemm_tile_choice(
        M, N, K, batch, cus, *(ctypes.byref(o) for o in out)))
    return tuple(o.value for o in out)


def sgemm_run_strided_batched(transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb,
                              strideB, beta, C, ldc, strideC, batch, stream=None) -> None:
    """`batch` general products, operands `stride*` floats apart."""
    _check("sgemm_run_strided_batched", load_library().sgemm_run_strided_batched(
        int(transA), int(transB), M, N, K, float(alpha), _ptr(A), lda, strideA, _ptr(B), ldb,
        strideB, float(beta), _ptr(C), ldc, strideC, batch, _stream(stream)))


def sgemm_bf16x3_workspace_size(M, N, K) -> int:
    """Workspace bytes sgemm_run_bf16x3 needs (include/sgemm_bf16x3.h)."""
    r = load_library().sgemm_bf16x3_workspace_size(M, N, K)
    if r < 0:
        raise SgemmError("sgemm_bf16x3_workspace_size", int(r))
    return int(r)


def sgemm_run_bf16x3(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes,
                     stream=None) -> None:
    """C = A x B on the bfloat16 matrix cores (three-piece split)."""
    _check("sgemm_run_bf16x3", load_library().sgemm_run_bf16x3(
        M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(workspace), workspace_bytes,
        _stream(stream)))


def sgemm_run_bf16x3_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                        workspace, workspace_bytes, stream=None) -> None:
    """C = alpha op(A) op(B) + beta C on the bfloat16 matrix cores."""
    _check("sgemm_run_bf16x3_ex", load_library().sgemm_run_bf16x3_ex(
        int(transA), int(transB), M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb,
        float(beta), _ptr(C), ldc, _ptr(workspace), workspace_bytes, _stream(stream)))


def sgemm_run_bf16x3_ex_noalloc(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                stream=None) -> None:
    """sgemm_run_bf16x3_ex with the library-held split buffer (no workspace)."""
    _check("sgemm_run_bf16x3_ex_noalloc", load_library().sgemm_run_bf16x3_ex_noalloc(
        int(transA), int(transB), M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb,
        float(beta), _ptr(C), ldc, _stream(stream)))


def vector_add(n, A, B, C, stream=None) -> None:
    """C[i] = A[i] + B[i] for i < n (include/vector_add.h)."""
    _check("vector_add", load_library().vector_add(n, _ptr(A), _ptr(B), _ptr(C),
                                                   _stream(stream)))


def sgemm_mfma_ceiling(which, iters, out, out_len, stream=None) -> float:
    """Launch the register-only matrix-core loop; return its flop count."""
    flops = ctypes.c_double(0.0)
    _check("sgemm_mfma_ceiling", load_library().sgemm_mfma_ceiling(
        int(which), int(iters), _ptr(out), int(out_len), ctypes.byref(flops), _stream(stream)))
    return flops.value


def sgemm_phase_times(M, N, K, A, lda, B, ldb, C, ldc, times, times_len, stream=None) -> int:
    """sgemm_run with per-work-group phase timestamps in `times` (8 uint64
    per work-group; times=None only queries); returns the work-group count."""
    wgs = ctypes.c_int64(0)
    _check("sgemm_phase_times", load_library().sgemm_phase_times(
        M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(times), int(times_len),
        ctypes.byref(wgs), _stream(stream)))
    return wgs.value


def sgemm_mfma_probe(which, A, B, C, stream=None) -> None:
    _check("sgemm_mfma_probe", load_library().sgemm_mfma_probe(
        int(which), _ptr(A), _ptr(B), _ptr(C), _stream(stream)))


def sgemm_status_string(status: int) -> str:
    return load_library().sgemm_status_string(int(status)).decode()


def sgemm_variant_name(variant: int):
    s = load_library().sgemm_variant_name(int(variant))
    return s.decode() if s is not None else None


def matmul(A, B, out=None, variant=None, stream=None):
    """C = A @ B for 2-D float32 torch tensors on the GPU (row-major, unit
    column stride; row strides become the leading dimensions).  Allocates
    `out` with torch when it is not given."""
    import torch
    if A.dtype != torch.float32 or B.dtype != torch.float32:
        raise TypeError("A and B must be float32")
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shapes {tuple(A.shape)} x {tuple(B.shape)} do not chain")
    M, K = A.shape
    N = B.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    for name, t in (("A", A), ("B", B), ("out", out)):
        if t.dim() == 2 and t.shape[0] > 0 and t.shape[1] > 1 and t.stride(1) != 1:
            raise ValueError(f"{name} must have unit column stride")
    lda = max(A.stride(0), 1) if M > 0 else max(K, 1)
    ldb = max(B.stride(0), 1) if K > 0 else max(N, 1)
    ldc = max(out.stride(0), 1) if M > 0 else max(N, 1)
    if variant is None:
        sgemm_run(M, N, K, A, lda, B, ldb, out, ldc, stream)
    else:
        sgemm_run_variant(variant, M, N, K, A, lda, B, ldb, out, ldc, stream)
    return out
