"""Parity of the HIP path with the CPU oracle, through the C-ABI.

Every product here is computed by libsgemm on the GPU and compared element by
element with the double-precision oracle on the same seeded inputs:

* the tolerance |C - Cref| <= 1e-5 * sum_k |A(i,k) B(k,j)| + 1e-6 with C
  finite (C is pre-filled with NaN, so an entry never written fails);
* bit-exact agreement for small-integer inputs, where single precision is
  exact;
* at 8192^3, 4096 sampled entries against the oracle plus whole-matrix checks
  (every entry finite, a double-precision Freivalds check, and exact integer
  Freivalds checks on an integer-valued product).
"""
import numpy as np
import pytest

import dense_fp32_matrix_03_amd as sg
import oracle
from dense_fp32_matrix_03_amd import inputs
from tile_rule import _expected_tile

pytestmark = pytest.mark.gpu

MFMA_VARIANTS = ["mfma", "mfma_256", "mfma_128", "mfma_64", "mfma_staged", "mfma_unpadded",
                 "mfma_32", "mfma_dword", "mfma_32x64", "mfma_serial", "mfma_16", "mfma_64x96"]
VALU_VARIANTS = ["naive", "lds", "reg", "dbuf"]
ALL_VARIANTS = VALU_VARIANTS + MFMA_VARIANTS


@pytest.fixture(scope="module", autouse=True)
def library():
    sg.sgemm_create()
    yield
    sg.sgemm_destroy()


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


# C sits inside a NaN-filled buffer: GUARD_LEAD floats before its first
# element (an odd count, so C's base is 4-byte but not 16-byte aligned) and
# GUARD_ROWS rows of ldc floats after its last row.  A store outside the M x N
# block (rows >= M, columns in [N, ldc), or before the base) shows up as a
# guard or padding value that is no longer NaN.  Out-of-range positions must
# not be touched: textbook chapter "4. 矩阵乘法性能优化", section 三
# (boundary handling).
GUARD_LEAD = 37
GUARD_ROWS = 3


def _run(A, B, M, N, K, variant="mfma", ldc=None, lda=None, ldb=None):
    """Run one product on the GPU from host arrays; return C (M x ldc) on the
    host after checking that every float around the M x N block is still NaN."""
    import torch
    lda = A.shape[1] if lda is None else lda
    ldb = B.shape[1] if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    dA, dB = _dev(A), _dev(B)
    rows = max(M, 1)
    buf = torch.full((GUARD_LEAD + (rows + GUARD_ROWS) * ldc,), float("nan"),
                     dtype=torch.float32, device="cuda")
    sg.sgemm_run_variant(variant, M, N, K, dA, lda, dB, ldb, buf.data_ptr() + 4 * GUARD_LEAD,
                         ldc)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    _check_guards(host, M, N, ldc)
    return host[GUARD_LEAD:GUARD_LEAD + rows * ldc].reshape(rows, ldc)[:M]


def _check_guards(host, M, N, ldc):
    """Every float of `host` outside the M x N block that starts GUARD_LEAD
    floats in (row stride ldc) is NaN."""
    assert np.all(np.isnan(host[:GUARD_LEAD])), "a store landed before C's first element"
    rows = max(M, 1)
    tail = host[GUARD_LEAD + rows * ldc:]
    assert tail.size == GUARD_ROWS * ldc
    assert np.all(np.isnan(tail)), "a store landed after C's last row"
    body = host[GUARD_LEAD:GUARD_LEAD + rows * ldc].reshape(rows, ldc)
    assert np.all(np.isnan(body[:, N:])), "a store landed in C's padding columns"
    if M == 0:
        assert np.all(np.isnan(body)), "a product with M = 0 wrote C"


# -- layout probe ---------------------------------------------------------------

@pytest.mark.parametrize("which,m,k", [(0, 32, 2), (1, 16, 4)])
def test_mfma_probe_index_encoded(which, m, k):
    """A(i,k) = i + 100 k, B(k,j) = 1000 k - j: integers, so exact."""
    import torch
    A = np.array([[i + 100 * kk for kk in range(k)] for i in range(m)], dtype=np.float32)
    B = np.array([[1000 * kk - j for j in range(m)] for kk in range(k)], dtype=np.float32)
    dC = torch.full((m, m), float("nan"), dtype=torch.float32, device="cuda")
    sg.sgemm_mfma_probe(which, _dev(A), _dev(B), dC)
    torch.cuda.synchronize()
    Cref, _ = oracle.sgemm_f64(A, B)
    assert np.array_equal(dC.cpu().numpy().astype(np.float64), Cref)


@pytest.mark.parametrize("which,per_instr", [(0, 2 * 32 * 32 * 2), (1, 2 * 32 * 32 * 16)])
def test_mfma_ceiling_loop_runs(which, per_instr):
    """The register-only ceiling loop: flop count and finite per-thread sums."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.full((1024 * cus,), float("nan"), dtype=torch.float32, device="cuda")
    flops = sg.sgemm_mfma_ceiling(which, 50, out, out.numel())
    torch.cuda.synchronize()
    assert flops == per_instr * 8 * 50 * (4 * cus) * 4
    assert bool(torch.isfinite(out).all().item())
    with pytest.raises(sg.SgemmError):
        sg.sgemm_mfma_ceiling(which, 50, out, out.numel() - 1)


# -- the five workloads -----------------------------------------------------------

@pytest.mark.parametrize("w", inputs.WORKLOADS[:4], ids=lambda w: w.name)
def test_workload_tolerance(w):
    A, B = inputs.make_inputs(w)
    C = _run(A, B, w.M, w.N, w.K, ldc=w.ldc)
    Cref, Sabs = oracle.sgemm_f64(A, B, K=w.K, N=w.N)
    r = oracle.check(C[:, :w.N], Cref, Sabs)
    print(f"{w.name}: {r}")
    assert r.ok, str(r)
    assert r.usage < 0.05, f"tolerance usage {r.usage} suggests a precision defect"


@pytest.mark.parametrize("w", inputs.WORKLOADS[:4], ids=lambda w: w.name)
def test_workload_integer_exact(w):
    A, B = inputs.make_inputs(w, dist="int8range")
    C = _run(A, B, w.M, w.N, w.K, ldc=w.ldc)
    Cref, _ = oracle.sgemm_f64(A, B, K=w.K, N=w.N)
    assert np.array_equal(C[:, :w.N].astype(np.float64), Cref)


def _big():
    return inputs.WORKLOADS[4]


def test_8192_sampled_and_whole_matrix():
    import torch
    w = _big()
    A, B = inputs.make_inputs(w)
    C = _run(A, B, w.M, w.N, w.K)
    assert np.all(np.isfinite(C)), "an output entry was never written"
    I, J = inputs.sample_indices(w.M, w.N, w.seed)
    cref, sabs = oracle.entries_f64(A, B, I, J)
    r = oracle.check(C[I, J], cref, sabs)
    print(f"{w.name} sampled: {r}")
    assert r.ok, str(r)
    assert r.usage < 0.05
    ok, usage = oracle.freivalds(A, B, C, inputs.sign_vector(w.N, w.seed))
    print(f"{w.name} freivalds usage {usage:.3e}")
    assert ok
    del C
    torch.cuda.empty_cache()


def test_8192_integer_exact_whole_matrix():
    """Integer inputs in [-8, 8]: every partial sum is below 2^24, so C is exact
    and (C x) == A (B x) holds exactly in int64 for integer probe vectors."""
    w = _big()
    A, B = inputs.make_inputs(w, dist="int8range")
    C = _run(A, B, w.M, w.N, w.K)
    assert np.all(np.isfinite(C))
    Ci = C.astype(np.int64)
    assert np.array_equal(Ci.astype(np.float32), C)
    Ai, Bi = A.astype(np.int64), B.astype(np.int64)
    g = np.random.default_rng(99)
    for _ in range(3):
        x = g.integers(-1000, 1001, size=w.N, dtype=np.int64)
        assert np.array_equal(Ci @ x, Ai @ (Bi @ x))
    I, J = inputs.sample_indices(w.M, w.N, w.seed)
    cref, _ = oracle.entries_f64(A, B, I, J)
    assert np.array_equal(C[I, J].astype(np.float64), cref)


def test_8192_rank1_closed_form():
    """A(i,k) = u_i, B(k,j) = v_j: C(i,j) = K u_i v_j exactly, no oracle needed."""
    w = _big()
    g = np.random.default_rng(4)
    u = inputs.small_integers(g, (w.M,))
    v = inputs.small_integers(g, (w.N,))
    A = np.repeat(u[:, None], w.K, axis=1)
    B = np.repeat(v[None, :], w.K, axis=0)
    C = _run(A, B, w.M, w.N, w.K)
    expect = (w.K * np.outer(u.astype(np.int64), v.astype(np.int64))).astype(np.float32)
    assert np.array_equal(C, expect)


# -- every variant ------------------------------------------------------------------

@pytest.mark.parametrize("variant", ALL_VARIANTS)
@pytest.mark.parametrize("w", [inputs.WORKLOADS[0], inputs.WORKLOADS[3]], ids=lambda w: w.name)
def test_variant_tolerance(variant, w):
    A, B = inputs.make_inputs(w)
    C = _run(A, B, w.M, w.N, w.K, variant=variant, ldc=w.ldc)
    Cref, Sabs = oracle.sgemm_f64(A, B, K=w.K, N=w.N)
    r = oracle.check(C[:, :w.N], Cref, Sabs)
    assert r.ok, f"{variant}: {r}"
    assert r.usage < 0.05


@pytest.mark.parametrize("variant", ALL_VARIANTS)
def test_variant_integer_exact_1024(variant):
    w = inputs.WORKLOADS[1]
    A, B = inputs.make_inputs(w, dist="int8range")
    C = _run(A, B, w.M, w.N, w.K, variant=variant)
    Cref, _ = oracle.sgemm_f64(A, B)
    assert np.array_equal(C.astype(np.float64), Cref)


# -- edges: ragged shapes, padding, alignment ------------------------------------------

EDGE_DIMS = [1, 2, 3, 5, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def _edge_shapes(n, seed):
    g = np.random.default_rng(seed)
    return [tuple(int(x) for x in g.choice(EDGE_DIMS, 3)) for _ in range(n)]


@pytest.mark.parametrize("variant", ALL_VARIANTS)
def test_edge_shape_sweep(variant):
    for (M, N, K) in _edge_shapes(24, 7 + ALL_VARIANTS.index(variant)) + [(1, 1, 1), (257, 255, 3)]:
        g = np.random.default_rng(M * 65536 + N * 256 + K)
        A = inputs.uniform(g, (M, K))
        B = inputs.uniform(g, (K, N))
        C = _run(A, B, M, N, K, variant=variant)
        Cref, Sabs = oracle.sgemm_f64(A, B)
        r = oracle.check(C, Cref, Sabs)
        assert r.ok, f"{variant} M={M} N={N} K={K}: {r}"


# Extreme aspect ratios: a 4M-long dot product, tall and wide skinny products,
# an outer product (K = 1) and many tiles over a tiny K.
EXTREME_SHAPES = [(1, 1, 1 << 22), (2, 3, 1 << 20), (1 << 20, 3, 7), (5, 1 << 20, 9),
                  (4097, 4099, 1), (1 << 15, 1 << 9, 4)]


@pytest.mark.parametrize("variant", ["mfma", "mfma_256", "mfma_64", "mfma_staged", "mfma_32",
                                     "mfma_32x64", "mfma_serial", "mfma_16", "mfma_64x96"])
@pytest.mark.parametrize("shape", EXTREME_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_extreme_aspect_ratios(variant, shape):
    M, N, K = shape
    g = np.random.default_rng(M * 7 + N * 3 + K)
    A = inputs.uniform(g, (M, K))
    B = inputs.uniform(g, (K, N))
    print(f"{variant} M={M} N={N} K={K}", flush=True)
    C = _run(A, B, M, N, K, variant=variant)
    Cref, Sabs = oracle.sgemm_f64(A, B)
    r = oracle.check(C, Cref, Sabs)
    assert r.ok, f"{variant} M={M} N={N} K={K}: {r}"
    assert r.usage < 0.05, f"tolerance usage {r.usage}"


# Dimensions that are multiples of 4 (so the buffer-to-LDS path is taken) but
# of no tile size: ragged M/N tiles and a ragged last K slice.
DMA_DIMS = [4, 8, 12, 28, 36, 60, 68, 124, 132, 252, 260, 516]


@pytest.mark.parametrize("variant", ["mfma", "mfma_256", "mfma_128", "mfma_64", "mfma_unpadded",
                                     "mfma_32", "mfma_dword", "mfma_32x64", "mfma_serial",
                                     "mfma_16", "mfma_64x96"])
def test_buffer_to_lds_edge_sweep(variant):
    g0 = np.random.default_rng(53 + MFMA_VARIANTS.index(variant))
    shapes = [tuple(int(x) for x in g0.choice(DMA_DIMS, 3)) for _ in range(20)]
    for (M, N, K) in shapes + [(4, 4, 4), (516, 260, 36)]:
        g = np.random.default_rng(M * 65536 + N * 256 + K)
        A = inputs.uniform(g, (M, K))
        B = inputs.uniform(g, (K, N))
        C = _run(A, B, M, N, K, variant=variant)
        Cref, Sabs = oracle.sgemm_f64(A, B)
        r = oracle.check(C, Cref, Sabs)
        assert r.ok, f"{variant} M={M} N={N} K={K}: {r}"


@pytest.mark.parametrize("w,tile", [(inputs.WORKLOADS[1], "mfma_64"),
                                    (inputs.WORKLOADS[2], "mfma_128")],
                         ids=["1024", "2048"])
def test_load_paths_agree_bitwise(w, tile):
    """Buffer-to-LDS fetches with or without the LDS anti-conflict layout,
    16 or 4 bytes per lane, feed the same matrix-core sequence: at the tile
    the shape selects they give identical bits.  The register-staged kernel
    has no k split, so it matches them at 128 x 128 (2048^3) and meets the
    tolerance at 64 x 64, whose buffer-to-LDS form splits K over two sets of
    waves (1024^3)."""
    import torch
    A, B = inputs.make_inputs(w)
    dA, dB = _dev(A), _dev(B)
    outs = {}
    for variant in ("mfma", tile, "mfma_staged", "mfma_unpadded", "mfma_dword"):
        dC = torch.full((w.M, w.N), float("nan"), dtype=torch.float32, device="cuda")
        sg.sgemm_run_variant(variant, w.M, w.N, w.K, dA, w.K, dB, w.N, dC, w.N)
        torch.cuda.synchronize()
        outs[variant] = dC.cpu().numpy()
    same = ["mfma", tile, "mfma_unpadded", "mfma_dword"]
    if tile == "mfma_128":
        same.append("mfma_staged")
    else:
        Cref, Sabs = oracle.sgemm_f64(A, B)
        r = oracle.check(outs["mfma_staged"], Cref, Sabs)
        assert r.ok and r.usage < 0.05, str(r)
    for v in same[1:]:
        assert outs[v].tobytes() == outs["mfma"].tobytes(), v


@pytest.mark.parametrize("variant", ["mfma", "mfma_256", "mfma_64", "mfma_staged", "lds", "reg",
                                     "dbuf", "mfma_32", "mfma_dword", "mfma_32x64", "mfma_16",
                                     "mfma_64x96"])
def test_padded_leading_dimensions(variant):
    """NaN in the padding of A and B must not reach C; C's padding is untouched."""
    M, N, K = 200, 136, 72
    g = np.random.default_rng(31)
    # ld % 4 == 0: the buffer-to-LDS path reads around NaN padding
    A = inputs.padded(inputs.uniform(g, (M, K)), K + 12)
    B = inputs.padded(inputs.uniform(g, (K, N)), N + 8)
    C = _run(A, B, M, N, K, variant=variant, ldc=N + 20)
    Cref, Sabs = oracle.sgemm_f64(A, B, K=K, N=N)
    r = oracle.check(C[:, :N], Cref, Sabs)
    assert r.ok, str(r)
    assert np.all(np.isnan(C[:, N:])), "C padding columns were written"


@pytest.mark.parametrize("variant", ["mfma", "mfma_128", "lds", "dbuf", "mfma_16", "mfma_64x96"])
def test_misaligned_pointers(variant):
    """Operands that start 4 or 12 bytes past a 16-byte boundary: 16-byte
    buffer-to-LDS loads from dword-aligned addresses, 4-byte loads in the
    other kernels."""
    import torch
    M, N, K = 130, 100, 68
    g = np.random.default_rng(37)
    A = inputs.uniform(g, (M, K))
    B = inputs.uniform(g, (K, N))
    bufA = _dev(np.concatenate([np.zeros(1, np.float32), A.ravel()]))
    bufB = _dev(np.concatenate([np.zeros(3, np.float32), B.ravel()]))
    dC = torch.full((GUARD_LEAD + (M + GUARD_ROWS) * N,), float("nan"), dtype=torch.float32,
                    device="cuda")
    sg.sgemm_run_variant(variant, M, N, K, bufA.data_ptr() + 4, K, bufB.data_ptr() + 12, N,
                         dC.data_ptr() + 4 * GUARD_LEAD, N)
    torch.cuda.synchronize()
    host = dC.cpu().numpy()
    _check_guards(host, M, N, N)
    C = host[GUARD_LEAD:GUARD_LEAD + M * N].reshape(M, N)
    Cref, Sabs = oracle.sgemm_f64(A, B)
    r = oracle.check(C, Cref, Sabs)
    assert r.ok, str(r)



def _unaligned_rows(A, lda, shift):
    """A's rows lda floats apart, `shift` floats into a NaN-filled device
    buffer (NaN in the padding past K and after the last row); returns the
    buffer and the byte address of A's first element."""
    M, K = A.shape
    host = np.full(shift + M * lda + 8, np.nan, np.float32)
    host[shift:shift + M * lda].reshape(M, lda)[:, :K] = A
    buf = _dev(host)
    return buf, buf.data_ptr() + 4 * shift


def _run_at(variant, M, N, K, a_ptr, lda, dB):
    """One product with A given by address; C inside NaN guards, checked."""
    import torch
    dC = torch.full((GUARD_LEAD + (M + GUARD_ROWS) * N,), float("nan"), dtype=torch.float32,
                    device="cuda")
    sg.sgemm_run_variant(variant, M, N, K, a_ptr, lda, dB, N, dC.data_ptr() + 4 * GUARD_LEAD, N)
    torch.cuda.synchronize()
    host = dC.cpu().numpy()
    _check_guards(host, M, N, N)
    return host[GUARD_LEAD:GUARD_LEAD + M * N].reshape(M, N)


# A's rows off the 16-byte grid (an odd lda, or a base 4, 8 or 12 bytes past
# it) with K % 4 = 0, 1, 2 and 3, on the shapes where sgemm_run takes each
# buffer-to-LDS configuration: the ragged workload's 64 x 96 tile, 32 x 64,
# 64 x 64 in two k sets (32- and 64-float slices), 32 x 32, 128 x 128, and
# an odd-sized product.  (M, N, K, lda, shift in floats.)
UNALIGNED_ROWS = [(1000, 1500, 777, 777, 0), (1000, 1500, 776, 777, 0), (800, 1280, 778, 781, 1),
                  (1024, 1024, 1024, 1025, 3), (896, 896, 1301, 1303, 2), (512, 512, 515, 517, 1),
                  (2048, 2048, 515, 515, 0), (129, 67, 45, 47, 1)]


@pytest.mark.parametrize("M,N,K,lda,shift", UNALIGNED_ROWS, ids=lambda v: str(v))
def test_unaligned_rows_take_16_byte_loads(M, N, K, lda, shift):
    """sgemm_run fetches rows of A that start off the 16-byte grid in 16-byte
    chunks, and a partial last K slice with K % 4 != 0 in 4-byte loads; both
    fill the LDS image that 4-byte loads fill, so the result has the bits of
    the forced 4-byte variant, meets the tolerance, and leaves C's
    surroundings untouched (NaN in A's padding never reaches C)."""
    g = np.random.default_rng(M + 3 * K + 7 * lda + shift)
    A = inputs.uniform(g, (M, K))
    B = inputs.uniform(g, (K, N))
    buf, a_ptr = _unaligned_rows(A, lda, shift)
    dB = _dev(B)
    C = _run_at("mfma", M, N, K, a_ptr, lda, dB)
    C4 = _run_at("mfma_dword", M, N, K, a_ptr, lda, dB)
    assert C.tobytes() == C4.tobytes()
    Cref, Sabs = oracle.sgemm_f64(A, B)
    r = oracle.check(C, Cref, Sabs)
    assert r.ok and r.usage < 0.05, str(r)


@pytest.mark.parametrize("variant", ["mfma_32", "mfma_32x64", "mfma_64", "mfma_64x96", "mfma_128",
                                     "mfma_256", "mfma_serial"])
@pytest.mark.parametrize("M,N,K,lda,shift", [(333, 257, 260, 263, 1), (600, 700, 777, 777, 0),
                                             (300, 520, 1299, 1301, 3)], ids=lambda v: str(v))
def test_unaligned_rows_every_tile(variant, M, N, K, lda, shift):
    """Each buffer-to-LDS tile gives the same bits from A's rows off the
    16-byte grid as from a copy whose rows are 16-byte aligned (the same
    tile, K slices and matrix-core sequence), and meets the tolerance."""
    g = np.random.default_rng(K * 5 + lda + shift)
    A = inputs.uniform(g, (M, K))
    B = inputs.uniform(g, (K, N))
    lda4 = (K + 3) // 4 * 4
    buf, a_ptr = _unaligned_rows(A, lda, shift)
    buf4, a4_ptr = _unaligned_rows(A, lda4, 0)
    dB = _dev(B)
    C = _run_at(variant, M, N, K, a_ptr, lda, dB)
    C4 = _run_at(variant, M, N, K, a4_ptr, lda4, dB)
    assert C.tobytes() == C4.tobytes()
    Cref, Sabs = oracle.sgemm_f64(A, B)
    r = oracle.check(C, Cref, Sabs)
    assert r.ok and r.usage < 0.05, str(r)

# sgemm_run's tile rule, restated: the tile that loses the least matrix-core
# time to partly filled rounds of work-groups and to tile area outside C
# (efficiency = M N batch / (rounds x CUs x tile area), rounds = ceil(tiles /
# CUs)), the larger one when two come within 3%; a tile whose launch would
# pass 2^32 work-items is out.
def test_expected_tile_on_256_cus():
    """The restated rule on 256 CUs picks the tiles measured best."""
    assert _expected_tile(256, 256, 256, 1, 256) == "mfma_16"
    assert _expected_tile(300, 260, 100, 1, 256) == "mfma_16"
    assert _expected_tile(768, 256, 256, 1, 256) == "mfma_32"    # 96 KiB per CU, 32 x 32 fills 3/4
    assert _expected_tile(512, 512, 64, 1, 256) == "mfma_16"
    assert _expected_tile(512, 512, 128, 1, 256) == "mfma_32"    # 64 KiB per CU
    assert _expected_tile(100, 3000, 64, 1, 256) == "mfma_16"    # 41 KiB per CU
    assert _expected_tile(640, 640, 64, 1, 256) == "mfma_32x64"  # 50 KiB per CU
    assert _expected_tile(512, 512, 256, 1, 256) == "mfma_32"    # 128 KiB, 32 x 32 fills the CUs
    assert _expected_tile(256, 256, 1024, 1, 256) == "mfma_16"   # at the traffic bound
    assert _expected_tile(384, 384, 512, 1, 256) == "mfma_32"    # over it
    assert _expected_tile(2048, 2048, 8, 1, 256) == "mfma_128"   # over 8 tiles per CU
    assert _expected_tile(512, 512, 512, 1, 256) == "mfma_32"
    assert _expected_tile(1000, 130, 1024, 1, 256) == "mfma_32"
    assert _expected_tile(1000, 130, 2048, 1, 256) == "mfma_32"
    assert _expected_tile(1000, 1500, 777, 1, 256) == "mfma_64x96"    # 256 tiles, one round
    assert _expected_tile(1000, 1700, 777, 1, 256) == "mfma_32"       # 288 tiles of 64 x 96
    assert _expected_tile(1024, 1536, 1024, 1, 256) == "mfma_64x96"
    assert _expected_tile(1024, 1024, 1024, 1, 256) == "mfma_64"
    assert _expected_tile(2048, 2048, 2048, 1, 256) == "mfma_128"
    assert _expected_tile(8192, 8192, 8192, 1, 256) == "mfma_256"
    assert _expected_tile(64, 64, 64, 1024, 256) == "mfma_64"


@pytest.mark.parametrize("M,N,K,batch", [
    (512, 512, 512, 1), (256, 256, 256, 1), (300, 260, 100, 1), (1000, 130, 2048, 1),
    (1024, 1024, 256, 1), (64, 64, 64, 256), (128, 128, 128, 8), (768, 1024, 512, 1),
    (832, 1024, 512, 1), (1000, 1500, 776, 1), (640, 640, 2048, 1), (3072, 3072, 64, 1),
    (768, 256, 256, 1), (256, 256, 1024, 1), (384, 384, 512, 1), (64, 64, 1024, 1),
    (512, 512, 64, 1)])
def test_tile_choice(M, N, K, batch):
    """sgemm_run takes the tile of the rule above on this device's CU count:
    its bits equal those of that forced tile (same K-slice rule), and both
    meet the oracle.  A batch is checked against the oracle on its first and
    last products."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tile = _expected_tile(M, N, K, batch, cus)
    g = np.random.default_rng(M + N + K + batch)
    A = inputs.uniform(g, (batch, M, K))
    B = inputs.uniform(g, (batch, K, N))
    dA, dB = _dev(A), _dev(B)
    outs = []
    for variant in ("mfma", tile):
        dC = torch.full((batch, M, N), float("nan"), dtype=torch.float32, device="cuda")
        if batch == 1:
            sg.sgemm_run_variant(variant, M, N, K, dA, K, dB, N, dC, N)
        else:
            sg.sgemm_run_strided_batched(0, 0, M, N, K, 1.0, dA, K, M * K, dB, N, K * N, 0.0,
                                         dC, N, M * N, batch)
        torch.cuda.synchronize()
        outs.append(dC.cpu().numpy())
        if batch > 1:
            break
    for b in sorted({0, batch - 1}):
        Cref, Sabs = oracle.sgemm_f64(A[b], B[b])
        r = oracle.check(outs[0][b], Cref, Sabs)
        assert r.ok, f"batch {b}: {r}"
        assert r.usage < 0.05
    if batch == 1:
        assert outs[0].tobytes() == outs[1].tobytes(), f"sgemm_run did not take {tile}"


def test_identity_gives_A_exactly():
    M, K = 300, 260
    g = np.random.default_rng(41)
    A = inputs.normal(g, (M, K))
    C = _run(A, np.eye(K, dtype=np.float32), M, K, K)
    assert np.array_equal(C, A)


def test_deterministic_bits():
    w = inputs.WORKLOADS[3]
    A, B = inputs.make_inputs(w)
    C1 = _run(A, B, w.M, w.N, w.K, ldc=w.ldc)
    C2 = _run(A, B, w.M, w.N, w.K, ldc=w.ldc)
    assert C1.tobytes() == C2.tobytes()


@pytest.mark.parametrize("M,N,K", [(512, 512, 512), (300, 260, 777), (1000, 130, 2048)])
def test_deterministic_bits_k_split_tile(M, N, K):
    """The k-split 32 x 32 tile adds its four partial sums in a fixed order:
    repeated calls, on two streams, give identical bits."""
    import torch
    g = np.random.default_rng(M + N + K)
    A = inputs.normal(g, (M, K))
    B = inputs.normal(g, (K, N))
    dA, dB = _dev(A), _dev(B)
    outs = []
    for _ in range(2):
        for s in (torch.cuda.current_stream(), torch.cuda.Stream()):
            dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
            s.wait_stream(torch.cuda.current_stream())  # the fill above comes first
            sg.sgemm_run(M, N, K, dA, K, dB, N, dC, N, s)
            s.synchronize()
            outs.append(dC.cpu().numpy().tobytes())
    assert all(o == outs[0] for o in outs[1:])
    assert not np.isnan(np.frombuffer(outs[0], dtype=np.float32)).any()


# Shapes on which sgemm_run takes each configuration on 256 CUs: the 16 x 16
# small-product tile (no LDS pipeline: the race-triage form runs it
# unchanged); 32 x 32 with 64- and 32-float K slices, 32 x 64 with both,
# 64 x 64 in two k sets with both, 64 x 64 in four waves, 128 x 128,
# 256 x 256; and a ragged K, an unaligned A (lda = 777) and an odd-sized
# product; and 64-float slices on the 64 x 64 tile in two k sets with a
# ragged K (1300) and with 4-byte A loads (lda = 1283).
RACE_TRIAGE_SHAPES = [(256, 256, 256, 256), (512, 512, 512, 512), (768, 768, 768, 768),
                      (640, 640, 2048, 2048),
                      (1000, 1500, 776, 776), (1000, 1500, 777, 777), (800, 1280, 777, 777),
                      (1024, 1024, 1024, 1024),
                      (1024, 1024, 2048, 2048), (896, 896, 1300, 1300), (832, 960, 1283, 1283),
                      (3072, 3072, 1024, 1024),
                      (2048, 2048, 2048, 2048), (4096, 4096, 1024, 1024), (300, 260, 100, 100),
                      (129, 67, 45, 45)]


@pytest.mark.parametrize("M,N,K,lda", RACE_TRIAGE_SHAPES, ids=lambda v: str(v))
def test_race_triage_schedule_gives_the_same_bits(M, N, K, lda):
    """SGEMM_VARIANT_MFMA_SERIAL computes every K slice with no load in flight
    and all waves in step, on sgemm_run's tile and matrix-core sequence: the
    two give identical bits (a difference would point to a race in the
    pipelined schedule), and the result meets the tolerance."""
    import torch
    g = np.random.default_rng(M * 3 + N * 5 + K * 7)
    A = inputs.padded(inputs.uniform(g, (M, K)), lda)
    B = inputs.uniform(g, (K, N))
    dA, dB = _dev(A), _dev(B)
    outs = {}
    for variant in ("mfma", "mfma_serial"):
        dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        sg.sgemm_run_variant(variant, M, N, K, dA, lda, dB, N, dC, N)
        torch.cuda.synchronize()
        outs[variant] = dC.cpu().numpy()
    assert outs["mfma_serial"].tobytes() == outs["mfma"].tobytes()
    if M * N * K <= 1 << 30:
        Cref, Sabs = oracle.sgemm_f64(A, B, K=K, N=N)
        r = oracle.check(outs["mfma"], Cref, Sabs)
        assert r.ok and r.usage < 0.05, str(r)


# -- the phase-timestamp diagnostic ----------------------------------------------------

@pytest.mark.parametrize("M,N,K,lda", [(256, 256, 256, 256), (1000, 1500, 777, 777),
                                       (1024, 1024, 2048, 2048), (2048, 2048, 96, 96),
                                       (100, 3000, 64, 64), (512, 512, 512, 512),
                                       (640, 640, 2048, 2048), (3072, 3072, 1024, 1024),
                                       (1024, 1024, 1024, 1024)])
def test_phase_times_diagnostic(M, N, K, lda):
    """sgemm_phase_times computes sgemm_run's bits (same tile and kernel
    code), and each work-group's timestamps are in order (start <= first
    slice landed <= last slice computed <= k sets reduced <= stores
    complete), with a tile record whose block count matches the launch and
    whose tile, K slice and k sets are what sgemm_tile_choice reports for
    this device's CU count."""
    import torch
    g = np.random.default_rng(M + N + K)
    A = inputs.padded(inputs.uniform(g, (M, K)), lda)
    B = inputs.uniform(g, (K, N))
    dA, dB = _dev(A), _dev(B)
    dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    dR = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    wgs = sg.sgemm_phase_times(M, N, K, dA, lda, dB, N, dC, N, None, 0)
    assert wgs > 0
    t = torch.zeros(8 * wgs, dtype=torch.int64, device="cuda")
    with pytest.raises(sg.SgemmError):
        sg.sgemm_phase_times(M, N, K, dA, lda, dB, N, dC, N, t, t.numel() - 1)
    assert sg.sgemm_phase_times(M, N, K, dA, lda, dB, N, dC, N, t, t.numel()) == wgs
    sg.sgemm_run(M, N, K, dA, lda, dB, N, dR, N)
    torch.cuda.synchronize()
    assert dC.cpu().numpy().tobytes() == dR.cpu().numpy().tobytes()
    q = t.cpu().numpy().reshape(wgs, 8)
    assert np.all(np.diff(q[:, :5], axis=1) >= 0), "phase timestamps out of order"
    assert np.all(q[:, 6] > q[:, 5]), "shader clock did not advance"
    tile = int(q[0, 7])
    assert np.all(q[:, 7] == tile)
    bm, bn, bk, ks = tile & 0xffff, (tile >> 16) & 0xffff, (tile >> 32) & 0xffff, tile >> 48
    assert -(-M // bm) * -(-N // bn) == wgs and bk % 16 == 0 and ks in (1, 2, 4)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert (bm, bn, bk, ks) == sg.sgemm_tile_choice(M, N, K, 1, cus)


# -- degenerate sizes and errors --------------------------------------------------------

def test_k_zero_writes_zeros():
    import torch
    dC = torch.full((5, 7), float("nan"), dtype=torch.float32, device="cuda")
    sg.sgemm_run(5, 6, 0, None, 1, None, 6, dC, 7)
    torch.cuda.synchronize()
    C = dC.cpu().numpy()
    assert np.array_equal(C[:, :6], np.zeros((5, 6), np.float32))
    assert np.all(np.isnan(C[:, 6]))


def test_m_or_n_zero_is_a_noop():
    import torch
    dC = torch.full((4, 4), float("nan"), dtype=torch.float32, device="cuda")
    sg.sgemm_run(0, 4, 4, None, 4, None, 4, dC, 4)
    sg.sgemm_run(4, 0, 4, None, 4, None, 1, dC, 4)
    torch.cuda.synchronize()
    assert np.all(np.isnan(dC.cpu().numpy()))


def test_errors_are_reported():
    import torch
    d = torch.zeros(16, device="cuda")
    with pytest.raises(sg.SgemmError) as e:
        sg.sgemm_run(4, 4, 4, d, 3, d, 4, d, 4)
    assert e.value.status == sg._C["SGEMM_ERR_INVALID_VALUE"]
    with pytest.raises(sg.SgemmError):
        sg.sgemm_run_variant(99, 4, 4, 4, d, 4, d, 4, d, 4)


def test_matmul_helper_and_streams():
    import torch
    g = np.random.default_rng(43)
    A = inputs.uniform(g, (96, 80))
    B = inputs.uniform(g, (80, 112))
    s = torch.cuda.Stream()
    dA, dB = _dev(A), _dev(B)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        dC = sg.matmul(dA, dB)
    s.synchronize()
    Cref, Sabs = oracle.sgemm_f64(A, B)
    assert oracle.check(dC.cpu().numpy(), Cref, Sabs).ok


def test_concurrent_streams():
    """Products of different shapes (so different tiles) on four streams at
    once, three rounds: the library keeps no per-call state."""
    import torch
    shapes = [(512, 384, 256), (1000, 1500, 777), (256, 256, 1024), (2048, 256, 64)]
    g = np.random.default_rng(47)
    cases = []
    for M, N, K in shapes:
        A = inputs.uniform(g, (M, K))
        B = inputs.uniform(g, (K, N))
        Cref, Sabs = oracle.sgemm_f64(A, B)
        cases.append((M, N, K, _dev(A), _dev(B), Cref, Sabs))
    streams = [torch.cuda.Stream() for _ in shapes]
    torch.cuda.synchronize()
    for _ in range(3):
        outs = []
        for (M, N, K, dA, dB, _, _), s in zip(cases, streams):
            with torch.cuda.stream(s):
                dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
                for _ in range(4):
                    sg.sgemm_run(M, N, K, dA, K, dB, N, dC, N, s)
            outs.append(dC)
        torch.cuda.synchronize()
        for (M, N, K, _, _, Cref, Sabs), dC in zip(cases, outs):
            r = oracle.check(dC.cpu().numpy(), Cref, Sabs)
            assert r.ok, f"{M}x{N}x{K}: {r}"


def test_host_threads():
    """Four host threads, each with its own stream, call sgemm_run (ctypes
    drops the GIL for the call) on different shapes; every result equals the
    single-threaded result bit for bit, and that one meets the oracle."""
    import threading

    import torch
    shapes = [(512, 384, 256), (1000, 1500, 777), (256, 256, 1024), (2048, 256, 64)]
    g = np.random.default_rng(59)
    cases = []
    for M, N, K in shapes:
        A = inputs.uniform(g, (M, K))
        B = inputs.uniform(g, (K, N))
        ref = _run(A, B, M, N, K)
        Cref, Sabs = oracle.sgemm_f64(A, B)
        assert oracle.check(ref, Cref, Sabs).ok
        cases.append((M, N, K, _dev(A), _dev(B), ref))
    torch.cuda.synchronize()
    errors = []
    results = [None] * len(cases)

    def worker(i):
        try:
            M, N, K, dA, dB, _ = cases[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
            for _ in range(25):
                sg.sgemm_run(M, N, K, dA, K, dB, N, dC, N, s)
            s.synchronize()
            results[i] = dC.cpu().numpy()
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    for (M, N, K, _, _, ref), out in zip(cases, results):
        assert out.tobytes() == ref.tobytes(), f"{M}x{N}x{K}"


def test_leading_dimension_past_32_bit_offsets():
    """lda = 2^30 + 8: a 32-row slice of A spans more than a buffer
    descriptor's 2 GiB, so sgemm_run (on the 32 x 32 tile: K = 1100 is past
    the 16 x 16 tile's K) falls back to the register-staged kernel (64-bit
    addressing); the general entry point reports SGEMM_ERR_TOO_LARGE, the
    16 x 16 small-product kernel (64-bit addressing, no buffer descriptors)
    and the bfloat16-split path (which reads A in its own split kernel)
    compute it."""
    import torch
    M, N, K, lda = 3, 48, 1100, (1 << 30) + 8
    g = np.random.default_rng(53)
    A = inputs.uniform(g, (M, K))
    B = inputs.uniform(g, (K, N))
    big = torch.full(((M - 1) * lda + K,), float("nan"), dtype=torch.float32, device="cuda")
    for i in range(M):
        big[i * lda:i * lda + K] = torch.from_numpy(A[i]).cuda()
    dB = _dev(B)
    Cref, Sabs = oracle.sgemm_f64(A, B)
    dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    sg.sgemm_run(M, N, K, big, lda, dB, N, dC, N)
    torch.cuda.synchronize()
    assert oracle.check(dC.cpu().numpy(), Cref, Sabs).ok
    with pytest.raises(sg.SgemmError) as e:
        sg.sgemm_run_ex(0, 0, M, N, K, 1.0, big, lda, dB, N, 0.0, dC, N)
    assert e.value.status == sg._C["SGEMM_ERR_TOO_LARGE"]
    with pytest.raises(sg.SgemmError) as e:  # the race-triage form has no register-staged kernel
        sg.sgemm_run_variant("mfma_serial", M, N, K, big, lda, dB, N, dC, N)
    assert e.value.status == sg._C["SGEMM_ERR_TOO_LARGE"]
    dC.fill_(float("nan"))
    sg.sgemm_run_variant("mfma_16", M, N, K, big, lda, dB, N, dC, N)
    torch.cuda.synchronize()
    assert oracle.check(dC.cpu().numpy(), Cref, Sabs).ok
    nbytes = sg.sgemm_bf16x3_workspace_size(M, N, K)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dC.fill_(float("nan"))
    sg.sgemm_run_bf16x3(M, N, K, big, lda, dB, N, dC, N, ws, nbytes)
    torch.cuda.synchronize()
    assert oracle.check(dC.cpu().numpy(), Cref, Sabs).ok
    del big
    torch.cuda.empty_cache()
