"""Seeded synthetic inputs for the single-precision product C = A x B.

This module only draws numbers and lays them out; it contains none of the
product's arithmetic.  The GPU path and the CPU oracle both take their inputs
from here, so both always see the same bytes.

Workloads.  The pages compare square single-precision products of
1024 .. 8192 (the textbook chapter "4. 矩阵乘法性能优化", section 五, suggests
1024^3 and 2048^3; the blog "【infra之路】03_动手写 CUDA Kernel" uses 2048^2; the
article "硬件加速原理：CUDA核函数优化矩阵乘法的内存访问模式", section "测试环境与方法",
sweeps 1024^2 .. 8192^2).  No dataset is involved: the matrices are i.i.d.
draws, exactly as the pages fill theirs with pseudo-random values.

Generator: numpy's PCG64 via ``np.random.default_rng(seed)``.  A is drawn
first, then B.  Uniform[-1, 1) values are ``2 * U - 1`` with U a float32
uniform on [0, 1): U is a multiple of 2^-24, so 2U - 1 is a multiple of 2^-23
inside [-1, 1) and exactly representable.  Normal values are numpy's float32
standard normal.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dist: str          # "uniform" on [-1, 1) or "normal" (0, 1)
    seed: int
    lda: int
    ldb: int
    ldc: int
    check: str         # "full" or "sampled"

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def min_bytes(self) -> int:
        # A and B read once, C written once (C is never read).
        return 4 * (self.M * self.K + self.K * self.N + self.M * self.N)


def _sq(n, seed, check="full"):
    return Workload(f"sgemm_{n}x{n}x{n}_uniform_seed{seed}", n, n, n, "uniform", seed,
                    n, n, n, check)


# The five workloads, in order: small (the oracle's quick case), 1024^3,
# 2048^3 (the pages' main comparison size), a ragged shape whose A rows are
# not 16-byte aligned, and 8192^3.
WORKLOADS = (
    _sq(256, 0),
    _sq(1024, 1),
    _sq(2048, 2),
    Workload("sgemm_1000x1500x777_normal_seed3", 1000, 1500, 777, "normal", 3,
             777, 1500, 1500, "full"),
    _sq(8192, 4, check="sampled"),
)
BY_NAME = {w.name: w for w in WORKLOADS}


def uniform(g: np.random.Generator, shape) -> np.ndarray:
    """float32 i.i.d. uniform on [-1, 1), exactly representable values."""
    u = g.random(shape, dtype=np.float32)
    return (np.float32(2.0) * u - np.float32(1.0)).astype(np.float32, copy=False)


def normal(g: np.random.Generator, shape) -> np.ndarray:
    return g.standard_normal(shape, dtype=np.float32)


def small_integers(g: np.random.Generator, shape, lo: int = -8, hi: int = 8) -> np.ndarray:
    """Integers in [lo, hi] stored as float32 (exact)."""
    return g.integers(lo, hi + 1, size=shape).astype(np.float32)


def draw(g: np.random.Generator, dist: str, shape) -> np.ndarray:
    if dist == "uniform":
        return uniform(g, shape)
    if dist == "normal":
        return normal(g, shape)
    if dist == "int8range":
        return small_integers(g, shape)
    raise ValueError(f"unknown distribution {dist!r}")


def padded(x: np.ndarray, ld: int, fill=np.nan) -> np.ndarray:
    """Copy x (rows x cols) into a (rows x ld) buffer whose extra columns hold fill."""
    rows, cols = x.shape
    if ld < cols:
        raise ValueError(f"ld={ld} < cols={cols}")
    out = np.full((rows, ld), fill, dtype=np.float32)
    out[:, :cols] = x
    return out


def make_inputs(w: Workload, dist: str | None = None):
    """Return (A, B) as float32 arrays of shapes (M, lda) and (K, ldb).

    Columns beyond K (for A) and N (for B) are NaN so that any read of
    padding shows up in the result.  ``dist`` overrides the workload's
    distribution (e.g. "int8range" for the exactness cases).
    """
    g = np.random.default_rng(w.seed)
    d = w.dist if dist is None else dist
    A = draw(g, d, (w.M, w.K))
    B = draw(g, d, (w.K, w.N))
    if w.lda != w.K:
        A = padded(A, w.lda)
    if w.ldb != w.N:
        B = padded(B, w.ldb)
    return A, B


# Fixed sample points for the 8192^3 check: the four corners and the
# 256-tile seams {127, 128, 255, 256}^2, then uniform random entries.
_SEAMS = (127, 128, 255, 256)


def sample_indices(M: int, N: int, seed: int, n: int = 4096):
    """Return (I, J) int64 arrays of n entries to check for an M x N product."""
    fixed = [(0, 0), (0, N - 1), (M - 1, 0), (M - 1, N - 1)]
    fixed += [(i, j) for i in _SEAMS for j in _SEAMS if i < M and j < N]
    fixed = fixed[:n]
    g = np.random.default_rng(10_000 + seed)
    rest = n - len(fixed)
    I = np.concatenate([np.array([p[0] for p in fixed], dtype=np.int64),
                        g.integers(0, M, size=rest, dtype=np.int64)])
    J = np.concatenate([np.array([p[1] for p in fixed], dtype=np.int64),
                        g.integers(0, N, size=rest, dtype=np.int64)])
    return I, J


def sign_vector(n: int, seed: int) -> np.ndarray:
    """A +-1 probe vector for the whole-matrix (Freivalds) check."""
    g = np.random.default_rng(20_000 + seed)
    return np.where(g.random(n) < 0.5, -1.0, 1.0)


# Vector addition (the blog's experiment 1): n = 2^24 floats, A[i] = sin(i)^2
# and B[i] = cos(i)^2 with i converted to float and single-precision sine and
# cosine, so every exact sum is close to 1.
VECTOR_ADD_N = 1 << 24


def vector_add_inputs(n: int = VECTOR_ADD_N, kind: str = "sincos", seed: int = 0):
    """Return (A, B), float32 arrays of n elements."""
    if kind == "sincos":
        x = np.arange(n, dtype=np.float32)
        s = np.sin(x)
        c = np.cos(x)
        return (s * s).astype(np.float32), (c * c).astype(np.float32)
    if kind == "uniform":
        g = np.random.default_rng(seed)
        return uniform(g, (n,)), uniform(g, (n,))
    raise ValueError(f"unknown vector-add input kind {kind!r}")
