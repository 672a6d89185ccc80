"""Double-precision CPU oracle for the single-precision product C = A x B.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The HIP library never
loads it and shares no source with it; the product path has no CPU fallback.

What is here:

* ``sgemm_f64`` / ``entries_f64`` -- thin ctypes wrappers around the plain C
  loops in ``oracle.c``: entry (i, j) is the ascending-k sum of the exact
  double products A(i,k) * B(k,j), plus the sum of their absolute values.
  The definition is the summation formula of the article "硬件加速原理：CUDA核函数
  优化矩阵乘法的内存访问模式", section "矩阵乘法的计算特性".
* ``entries_ex_f64`` -- selected entries of the general form, equal to
  ``sgemm_ex_f64``'s entry by entry (for products too large to compute whole).
* ``sgemm_ex_f64`` -- the general form C = alpha op(A) op(B) + beta C0 with
  optionally transposed operands; the same exact-product, ascending-k double
  sum, then alpha * sum + beta * C0, with scale |alpha| S + |beta| |C0|.
* ``check`` -- the per-element acceptance test
  |C - Cref| <= 1e-5 * sum_k |A(i,k) B(k,j)| + 1e-6, with C finite.
* ``freivalds`` -- a whole-matrix necessary condition of that test, used at
  sizes where the full oracle product is too slow: for a sign vector x,
  |(C x)_i - (A (B x))_i| <= 1e-5 (|A| (|B| |x|))_i + 1e-6 N.
* ``exact_products`` -- exact rational sums for tiny inputs (brute force).
* ``vector_add`` -- C[i] = A[i] + B[i] correctly rounded to float (the
  blog's experiment 1, "向量加法"), from ``oracle_vector_add`` in oracle.c.
* ``split_bf16x3`` -- the three bfloat16 pieces x0 + x1 + x2 = x, each the
  nearest 8-significant-bit value to what is left (``oracle_split_bf16x3``).

Matrices are passed as numpy float32 arrays of shape (rows, ld); the logical
column count is given separately, so columns ld > cols are padding that the
oracle never reads.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from fractions import Fraction

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

RTOL = 1e-5  # relative part of the per-element tolerance
ATOL = 1e-6  # absolute part of the per-element tolerance


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so next to it (plain gcc, no HIP)."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-o", _LIB + ".tmp", _SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, fp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
    lib.oracle_sgemm_f64.argtypes = [i64, i64, i64, fp, i64, fp, i64, dp, i64, dp, i64,
                                     ctypes.c_int]
    lib.oracle_sgemm_f64.restype = ctypes.c_int
    lib.oracle_entries_f64.argtypes = [i64, i64, i64, fp, i64, fp, i64, i64, fp, fp, dp, dp]
    lib.oracle_entries_f64.restype = ctypes.c_int
    lib.oracle_sgemm_ex_f64.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                        ctypes.c_double, fp, i64, fp, i64, ctypes.c_double,
                                        fp, i64, dp, i64, dp, i64, ctypes.c_int]
    lib.oracle_sgemm_ex_f64.restype = ctypes.c_int
    lib.oracle_entries_ex_f64.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                          ctypes.c_double, fp, i64, fp, i64, ctypes.c_double,
                                          fp, i64, i64, fp, fp, dp, dp]
    lib.oracle_entries_ex_f64.restype = ctypes.c_int
    lib.oracle_split_bf16x3.argtypes = [i64, fp, fp, fp, fp]
    lib.oracle_split_bf16x3.restype = ctypes.c_int
    lib.oracle_vector_add.argtypes = [i64, fp, fp, fp]
    lib.oracle_vector_add.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _as_f32(x: np.ndarray, rows: int, cols: int, name: str) -> tuple[np.ndarray, int]:
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError(f"{name} must be float32, got {x.dtype}")
    if x.ndim != 2 or x.shape[0] != rows or x.shape[1] < cols:
        raise ValueError(f"{name} has shape {x.shape}, need ({rows}, >= {cols})")
    if not x.flags.c_contiguous:
        x = np.ascontiguousarray(x)
    return x, max(1, x.shape[1])


def _ptr(x: np.ndarray):
    return x.ctypes.data_as(ctypes.c_void_p) if x.size else None


def sgemm_f64(A: np.ndarray, B: np.ndarray, K: int | None = None, N: int | None = None,
              want_sabs: bool = True, threads: int = 0):
    """Return (Cref, Sabs) as float64 arrays of shape (M, N).

    A has shape (M, lda) with lda >= K, B has shape (K, ldb) with ldb >= N.
    K defaults to A.shape[1] and N to B.shape[1].  Sabs is None when
    want_sabs is False.
    """
    M = A.shape[0]
    K = A.shape[1] if K is None else K
    N = B.shape[1] if N is None else N
    A, lda = _as_f32(A, M, K, "A")
    B, ldb = _as_f32(B, K, N, "B")
    C = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64) if want_sabs else None
    rc = _load().oracle_sgemm_f64(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), max(1, N),
                                  _ptr(S) if S is not None else None, max(1, N), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_sgemm_f64 rejected its arguments (rc={rc})")
    return C, S


def sgemm_ex_f64(transA: bool, transB: bool, M: int, N: int, K: int, alpha: float,
                 A: np.ndarray, B: np.ndarray, beta: float = 0.0, C0: np.ndarray | None = None,
                 threads: int = 0):
    """Return (Cref, Sabs) for C = alpha op(A) op(B) + beta C0 (float64, M x N).

    A is stored as an array of shape (K, lda) when transA else (M, lda); B as
    (N, ldb) when transB else (K, ldb).  C0 is float32 of shape (M, ldc0);
    it is not read when beta == 0.
    """
    A, lda = _as_f32(A, K if transA else M, M if transA else K, "A")
    B, ldb = _as_f32(B, N if transB else K, K if transB else N, "B")
    if beta != 0.0:
        C0, ldc0 = _as_f32(C0, M, N, "C0")
    else:
        C0, ldc0 = None, max(1, N)
    C = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_sgemm_ex_f64(int(transA), int(transB), M, N, K, float(alpha), _ptr(A),
                                     lda, _ptr(B), ldb, float(beta),
                                     _ptr(C0) if C0 is not None else None, ldc0, _ptr(C),
                                     max(1, N), _ptr(S), max(1, N), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_sgemm_ex_f64 rejected its arguments (rc={rc})")
    return C, S


def entries_f64(A: np.ndarray, B: np.ndarray, I, J, K: int | None = None,
                N: int | None = None):
    """Return (cref, sabs) for the listed entries (I[e], J[e])."""
    M = A.shape[0]
    K = A.shape[1] if K is None else K
    N = B.shape[1] if N is None else N
    A, lda = _as_f32(A, M, K, "A")
    B, ldb = _as_f32(B, K, N, "B")
    I = np.ascontiguousarray(I, dtype=np.int64)
    J = np.ascontiguousarray(J, dtype=np.int64)
    if I.shape != J.shape or I.ndim != 1:
        raise ValueError("I and J must be 1-D and of equal length")
    n = I.shape[0]
    c = np.empty(n, dtype=np.float64)
    s = np.empty(n, dtype=np.float64)
    rc = _load().oracle_entries_f64(M, N, K, _ptr(A), lda, _ptr(B), ldb, n, _ptr(I), _ptr(J),
                                    _ptr(c), _ptr(s))
    if rc != 0:
        raise ValueError(f"oracle_entries_f64 rejected its arguments (rc={rc})")
    return c, s


def entries_ex_f64(transA: bool, transB: bool, M: int, N: int, K: int, alpha: float,
                   A: np.ndarray, B: np.ndarray, I, J, beta: float = 0.0,
                   C0: np.ndarray | None = None):
    """(cref, sabs) of entries (I[e], J[e]) of alpha op(A) op(B) + beta C0;
    storage as for sgemm_ex_f64.  Equal, entry by entry, to sgemm_ex_f64."""
    A, lda = _as_f32(A, K if transA else M, M if transA else K, "A")
    B, ldb = _as_f32(B, N if transB else K, K if transB else N, "B")
    if beta != 0.0:
        C0, ldc0 = _as_f32(C0, M, N, "C0")
    else:
        C0, ldc0 = None, max(1, N)
    I = np.ascontiguousarray(I, dtype=np.int64)
    J = np.ascontiguousarray(J, dtype=np.int64)
    if I.shape != J.shape or I.ndim != 1:
        raise ValueError("I and J must be 1-D and of equal length")
    n = I.shape[0]
    c = np.empty(n, dtype=np.float64)
    s = np.empty(n, dtype=np.float64)
    rc = _load().oracle_entries_ex_f64(int(transA), int(transB), M, N, K, float(alpha), _ptr(A),
                                       lda, _ptr(B), ldb, float(beta),
                                       _ptr(C0) if C0 is not None else None, ldc0, n, _ptr(I),
                                       _ptr(J), _ptr(c), _ptr(s))
    if rc != 0:
        raise ValueError(f"oracle_entries_ex_f64 rejected its arguments (rc={rc})")
    return c, s


@dataclass
class CheckResult:
    ok: bool
    n_checked: int
    n_fail: int
    n_nonfinite: int
    usage: float          # max |C - Cref| / (RTOL * Sabs + ATOL): 1.0 is the bound
    worst: tuple          # index of the entry with the largest usage
    max_abs_err: float

    def __str__(self):
        return (f"ok={self.ok} checked={self.n_checked} fail={self.n_fail} "
                f"nonfinite={self.n_nonfinite} usage={self.usage:.3e} worst={self.worst} "
                f"max_abs_err={self.max_abs_err:.3e}")


def check(C, Cref, Sabs, rtol: float = RTOL, atol: float = ATOL) -> CheckResult:
    """Per-element acceptance test of a single-precision result C.

    Passes iff every C entry is finite and |C - Cref| <= rtol * Sabs + atol,
    evaluated in double.  ``usage`` reports how much of the bound the worst
    entry used.
    """
    C = np.asarray(C, dtype=np.float64)
    Cref = np.asarray(Cref, dtype=np.float64)
    Sabs = np.asarray(Sabs, dtype=np.float64)
    if C.shape != Cref.shape or C.shape != Sabs.shape:
        raise ValueError(f"shape mismatch {C.shape} {Cref.shape} {Sabs.shape}")
    finite = np.isfinite(C)
    n_nonfinite = int(C.size - np.count_nonzero(finite))
    err = np.abs(C - Cref)
    bound = rtol * Sabs + atol
    with np.errstate(invalid="ignore"):
        use = np.where(finite, err / bound, np.inf)
    n_fail = int(np.count_nonzero(~(use <= 1.0)))
    if C.size:
        w = int(np.argmax(use))
        worst = tuple(int(v) for v in np.unravel_index(w, C.shape))
        usage = float(use.flat[w])
        max_abs = float(np.max(np.where(finite, err, np.inf)))
    else:
        worst, usage, max_abs = (), 0.0, 0.0
    return CheckResult(ok=(n_fail == 0), n_checked=int(C.size), n_fail=n_fail,
                       n_nonfinite=n_nonfinite, usage=usage, worst=worst, max_abs_err=max_abs)


def freivalds(A: np.ndarray, B: np.ndarray, C: np.ndarray, x: np.ndarray,
              rtol: float = RTOL, atol: float = ATOL):
    """Whole-matrix check of C against A x B with one probe vector x.

    If every entry satisfies |C - AB| <= rtol |A||B| + atol, then for any x
    with |x_j| <= 1:  |(C x)_i - (A (B x))_i| <= rtol (|A| (|B| |x|))_i + atol N.
    Both sides are formed in double (library matrix-vector products, whose
    own rounding is ~1e-16 relative and far inside the bound).  Returns
    (ok, usage) where usage is the worst ratio of residual to bound.
    """
    M, K = A.shape[0], A.shape[1]
    N = C.shape[1]
    A64 = A[:, :K].astype(np.float64)
    B64 = B[:K, :N].astype(np.float64)
    x64 = np.asarray(x, dtype=np.float64)
    lhs = C.astype(np.float64) @ x64
    rhs = A64 @ (B64 @ x64)
    bound = rtol * (np.abs(A64) @ (np.abs(B64) @ np.abs(x64))) + atol * N
    res = np.abs(lhs - rhs)
    finite = bool(np.all(np.isfinite(lhs)))
    usage = float(np.max(res / bound)) if M else 0.0
    return (finite and usage <= 1.0), usage


def exact_products(A: np.ndarray, B: np.ndarray) -> list:
    """Exact rational matrix product of two small float arrays (brute force).

    Every float32 value is a dyadic rational, so Fraction(float(v)) is exact
    and the sum of products is computed with no rounding at all.
    """
    M, K = A.shape
    K2, N = B.shape
    assert K == K2
    FA = [[Fraction(float(A[i, k])) for k in range(K)] for i in range(M)]
    FB = [[Fraction(float(B[k, j])) for j in range(N)] for k in range(K)]
    return [[sum((FA[i][k] * FB[k][j] for k in range(K)), Fraction(0)) for j in range(N)]
            for i in range(M)]


def vector_add(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """C = A + B elementwise for 1-D float32 arrays, each sum correctly
    rounded to float32."""
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    if A.dtype != np.float32 or B.dtype != np.float32:
        raise TypeError("A and B must be float32")
    if A.ndim != 1 or A.shape != B.shape:
        raise ValueError(f"shapes {A.shape} and {B.shape} must be equal and 1-D")
    C = np.empty_like(A)
    rc = _load().oracle_vector_add(A.shape[0], _ptr(A), _ptr(B), _ptr(C))
    if rc != 0:
        raise ValueError(f"oracle_vector_add rejected its arguments (rc={rc})")
    return C


def split_bf16x3(x: np.ndarray):
    """Return (p0, p1, p2): uint16 bfloat16 bit patterns, same shape as x
    (float32), with x = p0 + p1 + p2 exactly for 2^-100 <= |x| <= 3.38e38."""
    x = np.ascontiguousarray(x)
    if x.dtype != np.float32:
        raise TypeError("x must be float32")
    flat = x.reshape(-1)
    out = [np.empty(flat.shape, dtype=np.uint16) for _ in range(3)]
    rc = _load().oracle_split_bf16x3(flat.shape[0], _ptr(flat), *(_ptr(o) for o in out))
    if rc != 0:
        raise ValueError(f"oracle_split_bf16x3 rejected its arguments (rc={rc})")
    return tuple(o.reshape(x.shape) for o in out)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """float32 values of bfloat16 bit patterns (the patterns are the high half)."""
    return (np.asarray(bits, dtype=np.uint32) << np.uint32(16)).view(np.float32)
