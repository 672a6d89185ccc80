"""Parity of the general form C = alpha op(A) op(B) + beta C and of strided
batches with the CPU oracle, through the C-ABI (sgemm_run_ex,
sgemm_run_strided_batched)."""
import numpy as np
import pytest

import dense_fp32_matrix_03_amd as sg
import oracle
from dense_fp32_matrix_03_amd import inputs

pytestmark = pytest.mark.gpu

LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]
LAYOUT_IDS = ["NN", "NT", "TN", "TT"]


@pytest.fixture(scope="module", autouse=True)
def library():
    sg.sgemm_create()
    yield
    sg.sgemm_destroy()


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _stored(g, ta, tb, M, N, K, dist="uniform"):
    A = inputs.draw(g, dist, (K, M) if ta else (M, K))
    B = inputs.draw(g, dist, (N, K) if tb else (K, N))
    return A, B


def _run_ex(ta, tb, M, N, K, alpha, A, B, beta, C0):
    """C0: float32 host array (M x ldc) or None for a NaN-filled C."""
    import torch
    dA, dB = _dev(A), _dev(B)
    if C0 is None:
        dC = torch.full((max(M, 1), max(N, 1)), float("nan"), dtype=torch.float32, device="cuda")
    else:
        dC = _dev(C0)
    ldc = dC.shape[1]
    sg.sgemm_run_ex(ta, tb, M, N, K, alpha, dA, A.shape[1], dB, B.shape[1], beta, dC, ldc)
    torch.cuda.synchronize()
    return dC.cpu().numpy()


@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (-1.5, 0.0), (0.5, 2.0), (1.0, -1.0)])
@pytest.mark.parametrize("shape", [(256, 256, 256), (1000, 1500, 777), (65, 130, 33)],
                         ids=lambda s: "x".join(map(str, s)))
def test_general_tolerance(ta, tb, alpha, beta, shape):
    M, N, K = shape
    g = np.random.default_rng(M + N + K + int(ta) * 2 + int(tb))
    A, B = _stored(g, ta, tb, M, N, K, "normal" if M == 1000 else "uniform")
    C0 = inputs.uniform(g, (M, N)) if beta != 0.0 else None
    C = _run_ex(ta, tb, M, N, K, alpha, A, B, beta, C0)
    Cref, Sabs = oracle.sgemm_ex_f64(ta, tb, M, N, K, alpha, A, B, beta, C0)
    r = oracle.check(C[:, :N], Cref, Sabs)
    assert r.ok, f"{ta}{tb} a={alpha} b={beta} {shape}: {r}"
    assert r.usage < 0.05


@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=LAYOUT_IDS)
def test_general_integer_exact_2048(ta, tb):
    M = N = K = 2048
    g = np.random.default_rng(97)
    A, B = _stored(g, ta, tb, M, N, K, "int8range")
    C0 = inputs.small_integers(g, (M, N), -50, 50)
    C = _run_ex(ta, tb, M, N, K, 2.0, A, B, -3.0, C0)
    Cref, _ = oracle.sgemm_ex_f64(ta, tb, M, N, K, 2.0, A, B, -3.0, C0)
    assert np.array_equal(C.astype(np.float64), Cref)


@pytest.mark.parametrize("ta,tb", LAYOUTS[1:], ids=LAYOUT_IDS[1:])
@pytest.mark.parametrize("shape", [(1024, 1024, 1024), (1000, 1500, 780), (300, 260, 100),
                                   (1000, 1500, 777), (332, 261, 101)],
                         ids=lambda s: "x".join(map(str, s)))
def test_transposed_storage_gives_identical_bits(ta, tb, shape):
    """The matrix-core sequence does not depend on how an operand is stored:
    op(A) op(B) from transposed copies equals the plain product bit for bit."""
    import torch
    M, N, K = shape
    g = np.random.default_rng(101)
    A = inputs.uniform(g, (M, K))
    B = inputs.uniform(g, (K, N))
    plain = _run_ex(False, False, M, N, K, 1.0, A, B, 0.0, None)
    As = np.ascontiguousarray(A.T) if ta else A
    Bs = np.ascontiguousarray(B.T) if tb else B
    other = _run_ex(ta, tb, M, N, K, 1.0, As, Bs, 0.0, None)
    assert plain.tobytes() == other.tobytes()
    # and the general entry point with alpha = 1, beta = 0 is sgemm_run
    dA, dB = _dev(A), _dev(B)
    dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    sg.sgemm_run(M, N, K, dA, K, dB, N, dC, N)
    torch.cuda.synchronize()
    assert dC.cpu().numpy().tobytes() == plain.tobytes()


EDGE = [1, 3, 4, 5, 31, 32, 33, 63, 64, 65, 127, 129, 255, 257]


@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=LAYOUT_IDS)
def test_general_edge_sweep(ta, tb):
    g0 = np.random.default_rng(107 + 2 * int(ta) + int(tb))
    for _ in range(16):
        M, N, K = (int(x) for x in g0.choice(EDGE, 3))
        g = np.random.default_rng(M * 65536 + N * 256 + K)
        A, B = _stored(g, ta, tb, M, N, K)
        C0 = inputs.uniform(g, (M, N))
        C = _run_ex(ta, tb, M, N, K, 0.75, A, B, 1.25, C0)
        Cref, Sabs = oracle.sgemm_ex_f64(ta, tb, M, N, K, 0.75, A, B, 1.25, C0)
        r = oracle.check(C, Cref, Sabs)
        assert r.ok, f"{ta}{tb} M={M} N={N} K={K}: {r}"


@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("pad_a,pad_b", [(0, 3), (1, 0), (4, 8), (5, 7)])
def test_padded_leading_dimensions(ta, tb, pad_a, pad_b):
    """Stored operands with NaN-filled columns past their stored width; the
    widths are multiples of 4, so pads of 0, 4 and 8 keep 16-byte loads and
    the odd pads force 4-byte ones.  A NaN ever read would reach C."""
    M, N, K = 132, 96, 76
    g = np.random.default_rng(149 + 16 * pad_a + pad_b + 2 * int(ta) + int(tb))
    A, B = _stored(g, ta, tb, M, N, K)
    A = inputs.padded(A, A.shape[1] + pad_a)
    B = inputs.padded(B, B.shape[1] + pad_b)
    C0 = inputs.uniform(g, (M, N))
    C = _run_ex(ta, tb, M, N, K, 1.25, A, B, -0.5, C0)
    Cref, Sabs = oracle.sgemm_ex_f64(ta, tb, M, N, K, 1.25, A, B, -0.5, C0)
    r = oracle.check(C, Cref, Sabs)
    assert r.ok, f"{ta}{tb} pads {pad_a},{pad_b}: {r}"


def test_alpha_zero_and_k_zero_scale_c():
    g = np.random.default_rng(109)
    C0 = inputs.uniform(g, (40, 50))
    A = np.full((40, 30), np.nan, dtype=np.float32)  # must not be read
    B = np.full((30, 50), np.nan, dtype=np.float32)
    C = _run_ex(False, False, 40, 50, 30, 0.0, A, B, -2.0, C0)
    assert np.array_equal(C, (-2.0 * C0).astype(np.float32))
    C = _run_ex(False, False, 40, 50, 0, 1.0, A[:, :1], B[:1], 0.5, C0)
    assert np.array_equal(C, (0.5 * C0).astype(np.float32))
    nanC = np.full((40, 50), np.nan, dtype=np.float32)
    C = _run_ex(False, False, 40, 50, 30, 0.0, A, B, 0.0, nanC)
    assert np.array_equal(C, np.zeros((40, 50), np.float32))


def test_beta_zero_ignores_nan_in_c():
    g = np.random.default_rng(113)
    A = inputs.uniform(g, (300, 200))
    B = inputs.uniform(g, (200, 400))
    C = _run_ex(False, False, 300, 400, 200, 1.5, A, B, 0.0, None)  # C starts as NaN
    Cref, Sabs = oracle.sgemm_ex_f64(False, False, 300, 400, 200, 1.5, A, B)
    assert oracle.check(C, Cref, Sabs).ok


@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=LAYOUT_IDS)
def test_strided_batched(ta, tb):
    """Five products with padded strides (NaN gaps), B shared by stride 0 in
    the NN case; every product checked against the oracle."""
    import torch
    M, N, K, batch = 96, 160, 72, 5
    g = np.random.default_rng(127 + 2 * int(ta) + int(tb))
    ar, ac = (K, M) if ta else (M, K)
    br, bc = (N, K) if tb else (K, N)
    sA, sB, sC = ar * ac + 44, (0 if not (ta or tb) else br * bc + 20), M * N + 12
    bufA = np.full(sA * batch + 64, np.nan, dtype=np.float32)
    bufB = np.full(max(sB * batch, br * bc) + 64, np.nan, dtype=np.float32)
    bufC = np.full(sC * batch + 64, np.nan, dtype=np.float32)
    As, Bs, C0s = [], [], []
    for b in range(batch):
        A = inputs.uniform(g, (ar, ac))
        bufA[b * sA:b * sA + ar * ac] = A.ravel()
        As.append(A)
        if sB or b == 0:
            Bm = inputs.uniform(g, (br, bc))
            bufB[b * sB:b * sB + br * bc] = Bm.ravel()
        Bs.append(bufB[b * sB:b * sB + br * bc].reshape(br, bc).copy())
        C0 = inputs.uniform(g, (M, N))
        bufC[b * sC:b * sC + M * N] = C0.ravel()
        C0s.append(C0)
    dA, dB, dC = _dev(bufA), _dev(bufB), _dev(bufC)
    sg.sgemm_run_strided_batched(ta, tb, M, N, K, 1.5, dA, ac, sA, dB, bc, sB, -0.5, dC, N, sC,
                                 batch)
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    for b in range(batch):
        C = out[b * sC:b * sC + M * N].reshape(M, N)
        Cref, Sabs = oracle.sgemm_ex_f64(ta, tb, M, N, K, 1.5, As[b], Bs[b], -0.5, C0s[b])
        r = oracle.check(C, Cref, Sabs)
        assert r.ok, f"batch {b}: {r}"
        assert np.all(np.isnan(out[b * sC + M * N:(b + 1) * sC])), "gap between C's written"


def test_batched_many_small_products():
    """256 products of 64^3 in one launch."""
    import torch
    M = N = K = 64
    batch = 256
    g = np.random.default_rng(131)
    A = inputs.uniform(g, (batch, M, K))
    B = inputs.uniform(g, (batch, K, N))
    dA, dB = _dev(A), _dev(B)
    dC = torch.full((batch, M, N), float("nan"), dtype=torch.float32, device="cuda")
    sg.sgemm_run_strided_batched(False, False, M, N, K, 1.0, dA, K, M * K, dB, N, K * N, 0.0,
                                 dC, N, M * N, batch)
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    for b in (0, 1, 127, 255):
        Cref, Sabs = oracle.sgemm_f64(A[b], B[b])
        assert oracle.check(out[b], Cref, Sabs).ok, b


def test_general_argument_errors():
    import torch
    d = torch.zeros(64, device="cuda")
    with pytest.raises(sg.SgemmError) as e:
        sg.sgemm_run_ex(2, 0, 4, 4, 4, 1.0, d, 4, d, 4, 0.0, d, 4)
    assert e.value.status == sg._C["SGEMM_ERR_INVALID_VALUE"]
    with pytest.raises(sg.SgemmError):  # transA: lda must cover M
        sg.sgemm_run_ex(1, 0, 8, 4, 4, 1.0, d, 4, d, 4, 0.0, d, 4)
    with pytest.raises(sg.SgemmError):  # negative stride
        sg.sgemm_run_strided_batched(0, 0, 4, 4, 4, 1.0, d, 4, -1, d, 4, 0, 0.0, d, 4, 16, 2)
    sg.sgemm_run_strided_batched(0, 0, 4, 4, 4, 1.0, d, 4, 0, d, 4, 0, 0.0, d, 4, 16, 0)  # no-op


@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=LAYOUT_IDS)
def test_general_8192_sampled(ta, tb):
    """The headline size in every layout, alpha = -0.75 and beta = 0.5: the
    sampled entries of the 8192^3 workload against the oracle, plus every
    entry finite."""
    import torch
    w = inputs.WORKLOADS[4]
    M = N = K = w.M
    g = np.random.default_rng(300 + 2 * int(ta) + int(tb))
    A, B = _stored(g, ta, tb, M, N, K)
    C0 = inputs.uniform(g, (M, N))
    dA, dB, dC = _dev(A), _dev(B), _dev(C0)
    sg.sgemm_run_ex(ta, tb, M, N, K, -0.75, dA, A.shape[1], dB, B.shape[1], 0.5, dC, N)
    torch.cuda.synchronize()
    C = dC.cpu().numpy()
    del dA, dB, dC
    torch.cuda.empty_cache()
    assert np.all(np.isfinite(C))
    I, J = inputs.sample_indices(M, N, w.seed)
    cref, sabs = oracle.entries_ex_f64(ta, tb, M, N, K, -0.75, A, B, I, J, 0.5, C0)
    r = oracle.check(C[I, J], cref, sabs)
    print(f"8192 {LAYOUT_IDS[2 * int(ta) + int(tb)]}: {r}")
    assert r.ok, str(r)
    assert r.usage < 0.05


@pytest.mark.parametrize("ta,tb", [(False, True), (True, False)], ids=["NT", "TN"])
def test_strided_batched_medium(ta, tb):
    """Six products of 1024 x 768 x 640 with padded strides and alpha/beta,
    each checked whole against the oracle."""
    import torch
    M, N, K, batch = 1024, 768, 640, 6
    g = np.random.default_rng(310 + int(ta))
    ar, ac = (K, M) if ta else (M, K)
    br, bc = (N, K) if tb else (K, N)
    sA, sB, sC = ar * ac + 128, br * bc + 64, M * N + 32
    A = [inputs.uniform(g, (ar, ac)) for _ in range(batch)]
    B = [inputs.uniform(g, (br, bc)) for _ in range(batch)]
    C0 = [inputs.uniform(g, (M, N)) for _ in range(batch)]
    bufA = np.full(sA * batch, np.nan, np.float32)
    bufB = np.full(sB * batch, np.nan, np.float32)
    bufC = np.full(sC * batch, np.nan, np.float32)
    for b in range(batch):
        bufA[b * sA:b * sA + ar * ac] = A[b].ravel()
        bufB[b * sB:b * sB + br * bc] = B[b].ravel()
        bufC[b * sC:b * sC + M * N] = C0[b].ravel()
    dA, dB, dC = _dev(bufA), _dev(bufB), _dev(bufC)
    sg.sgemm_run_strided_batched(ta, tb, M, N, K, 1.25, dA, ac, sA, dB, bc, sB, -1.0, dC, N, sC,
                                 batch)
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    for b in range(batch):
        Cref, Sabs = oracle.sgemm_ex_f64(ta, tb, M, N, K, 1.25, A[b], B[b], -1.0, C0[b])
        r = oracle.check(out[b * sC:b * sC + M * N].reshape(M, N), Cref, Sabs)
        assert r.ok, f"product {b}: {r}"
        assert np.all(np.isnan(out[b * sC + M * N:(b + 1) * sC]))
