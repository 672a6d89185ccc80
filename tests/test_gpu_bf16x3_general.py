"""The general form on the bfloat16 matrix cores (sgemm_run_bf16x3_ex),
C = alpha op(A) op(B) + beta C, against the oracle through the C-ABI.

* the split of a transposed source written to the workspace equals the
  oracle's three-piece split of op(A) and of op(B) transposed, bit for bit,
  for aligned and unaligned leading dimensions and ragged K;
* every layout and (alpha, beta) meets the tolerance of the single-precision
  path (|C - Cref| <= 1e-5 * Sabs + 1e-6, Sabs = sum_k |alpha a b| + |beta c|),
  at sizes that span several tiles and a ragged tail, and on 4096 sampled
  entries at 8192^3;
* the planes, and so the product, do not depend on how an operand is stored:
  transposed copies give the plain entry point's bits;
* integer-valued operands give exact results, and alpha == 0 or K == 0
  leaves beta C without reading A, B or the workspace.
"""
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


def _stored(g, ta, tb, M, N, K, dist="uniform", pad_a=0, pad_b=0):
    """Stored A and B (transposed shapes where ta / tb) with pad_* extra
    NaN columns each."""
    ar, ac = (K, M) if ta else (M, K)
    br, bc = (N, K) if tb else (K, N)
    A = inputs.padded(inputs.draw(g, dist, (ar, ac)), ac + pad_a)
    B = inputs.padded(inputs.draw(g, dist, (br, bc)), bc + pad_b)
    return A, B


def _run_ex(ta, tb, M, N, K, alpha, A, B, beta, C0, keep_workspace=False):
    """C0: float32 host array (M x ldc) or None for a NaN-filled C."""
    import torch
    dA, dB = _dev(A), _dev(B)
    if C0 is None:
        dC = torch.full((max(M, 1), max(N, 1)), float("nan"), dtype=torch.float32, device="cuda")
    else:
        dC = _dev(C0)
    nbytes = sg.sgemm_bf16x3_workspace_size(M, N, K)
    ws = torch.full((max(nbytes, 16) // 2,), 0x7fff, dtype=torch.int16, device="cuda")
    sg.sgemm_run_bf16x3_ex(ta, tb, M, N, K, alpha, dA, A.shape[1], dB, B.shape[1], beta, dC,
                           dC.shape[1], ws, nbytes)
    torch.cuda.synchronize()
    C = dC.cpu().numpy()
    if keep_workspace:
        return C, ws.cpu().numpy().view(np.uint16)
    return C


def _op(X, rows, cols, trans):
    """op(X) as a (rows x cols) float32 array from the stored X."""
    return np.ascontiguousarray(X[:cols, :rows].T if trans else X[:rows, :cols])


@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("M,N,K,pad_a,pad_b", [(96, 80, 100, 0, 0), (33, 70, 45, 3, 1),
                                               (256, 128, 64, 4, 0), (130, 67, 200, 1, 5)])
def test_workspace_holds_the_oracle_split(ta, tb, M, N, K, pad_a, pad_b):
    g = np.random.default_rng(M + N + K + 2 * int(ta) + int(tb))
    A, B = _stored(g, ta, tb, M, N, K, "normal", pad_a, pad_b)
    _, ws = _run_ex(ta, tb, M, N, K, 1.0, A, B, 0.0, None, keep_workspace=True)
    Kp = (K + 31) // 32 * 32
    wa = ws[:3 * M * Kp].reshape(3, M, Kp)
    wb = ws[3 * M * Kp:3 * (M + N) * Kp].reshape(3, N, Kp)
    Az = np.zeros((M, Kp), np.float32)
    Az[:, :K] = _op(A, M, K, ta)
    Bz = np.zeros((N, Kp), np.float32)
    Bz[:, :K] = _op(B, K, N, tb).T
    for pl, (pa, pb) in enumerate(zip(oracle.split_bf16x3(Az), oracle.split_bf16x3(Bz))):
        assert np.array_equal(wa[pl], pa), f"A plane {pl}"
        assert np.array_equal(wb[pl], pb), f"B plane {pl}"


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
    assert r.usage < 0.05, f"tolerance usage {r.usage} suggests a precision defect"


@pytest.mark.parametrize("ta,tb", LAYOUTS[1:], ids=LAYOUT_IDS[1:])
@pytest.mark.parametrize("shape", [(1024, 1024, 1024), (1000, 1500, 780), (300, 260, 100)],
                         ids=lambda s: "x".join(map(str, s)))
def test_transposed_storage_gives_identical_bits(ta, tb, shape):
    import torch
    M, N, K = shape
    g = np.random.default_rng(307)
    A = inputs.uniform(g, (M, K))
    B = inputs.uniform(g, (K, N))
    plain = _run_ex(False, False, M, N, K, 1.0, A, B, 0.0, None)
    As = np.ascontiguousarray(A.T) if ta else A
    Bs = np.ascontiguousarray(B.T) if tb else B
    other = _run_ex(ta, tb, M, N, K, 1.0, As, Bs, 0.0, None)
    assert plain.tobytes() == other.tobytes()
    # alpha = 1, beta = 0, no transposes is sgemm_run_bf16x3
    dA, dB = _dev(A), _dev(B)
    dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = sg.sgemm_bf16x3_workspace_size(M, N, K)
    ws = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda")
    sg.sgemm_run_bf16x3(M, N, K, dA, K, dB, N, dC, N, ws, nbytes)
    torch.cuda.synchronize()
    assert dC.cpu().numpy().tobytes() == plain.tobytes()


@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=LAYOUT_IDS)
def test_general_integer_exact_2048(ta, tb):
    M = N = K = 2048
    g = np.random.default_rng(311)
    A, B = _stored(g, ta, tb, M, N, K, "int8range")
    C0 = inputs.small_integers(g, (M, N), -50, 50)
    C = _run_ex(ta, tb, M, N, K, 2.0, A, B, -3.0, C0)
    Cref, _ = oracle.sgemm_ex_f64(ta, tb, M, N, K, 2.0, A, B, -3.0, C0)
    assert np.array_equal(C.astype(np.float64), Cref)


EDGE = [1, 3, 4, 5, 31, 32, 33, 63, 64, 65, 127, 129, 255, 257]


@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=LAYOUT_IDS)
def test_general_edge_sweep(ta, tb):
    g0 = np.random.default_rng(313 + 2 * int(ta) + int(tb))
    for _ in range(16):
        M, N, K = (int(x) for x in g0.choice(EDGE, 3))
        g = np.random.default_rng(M * 65536 + N * 256 + K)
        A, B = _stored(g, ta, tb, M, N, K, pad_a=int(g.integers(0, 3)),
                       pad_b=int(g.integers(0, 3)))
        C0 = inputs.uniform(g, (M, N))
        C = _run_ex(ta, tb, M, N, K, 0.75, A, B, 1.25, C0)
        Cref, Sabs = oracle.sgemm_ex_f64(ta, tb, M, N, K, 0.75, A, B, 1.25, C0)
        r = oracle.check(C, Cref, Sabs)
        assert r.ok, f"{ta}{tb} M={M} N={N} K={K}: {r}"


def test_8192_sampled_tt():
    """Both operands through the other split form, alpha and beta set."""
    import torch
    M = N = K = 8192
    g = np.random.default_rng(317)
    A, B = _stored(g, True, True, M, N, K, "uniform")
    C0 = inputs.uniform(g, (M, N))
    C = _run_ex(True, True, M, N, K, -1.5, A, B, 0.5, C0)
    assert np.all(np.isfinite(C))
    I, J = inputs.sample_indices(M, N, 317)
    cref, sabs = oracle.entries_ex_f64(True, True, M, N, K, -1.5, A, B, I, J, 0.5, C0)
    r = oracle.check(C[I, J], cref, sabs)
    print(f"8192 TT bf16x3 sampled: {r}")
    assert r.ok, str(r)
    assert r.usage < 0.05
    del C
    torch.cuda.empty_cache()


def test_alpha_zero_and_k_zero_scale_c():
    import torch
    g = np.random.default_rng(331)
    M, N = 40, 50
    C0 = inputs.uniform(g, (M, N))
    dC = _dev(C0)
    # alpha == 0: A, B and the workspace are not touched (null here)
    sg.sgemm_run_bf16x3_ex(True, False, M, N, 30, 0.0, None, M, None, N, -2.0, dC, N, None, 0)
    torch.cuda.synchronize()
    assert np.array_equal(dC.cpu().numpy(), (-2.0 * C0).astype(np.float32))
    dC = _dev(C0)
    sg.sgemm_run_bf16x3_ex(False, True, M, N, 0, 1.0, None, 1, None, 1, 0.5, dC, N, None, 0)
    torch.cuda.synchronize()
    assert np.array_equal(dC.cpu().numpy(), (0.5 * C0).astype(np.float32))
    dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    sg.sgemm_run_bf16x3_ex(False, False, M, N, 30, 0.0, None, 30, None, N, 0.0, dC, N, None, 0)
    torch.cuda.synchronize()
    assert np.array_equal(dC.cpu().numpy(), np.zeros((M, N), np.float32))


def test_beta_zero_ignores_nan_in_c():
    g = np.random.default_rng(337)
    A, B = _stored(g, True, False, 300, 400, 200)
    C = _run_ex(True, False, 300, 400, 200, 1.5, A, B, 0.0, None)  # C starts as NaN
    Cref, Sabs = oracle.sgemm_ex_f64(True, False, 300, 400, 200, 1.5, A, B)
    assert oracle.check(C, Cref, Sabs).ok
