"""Seeded random cases of the general form against the oracle.

Each case draws a layout, sizes, alpha and beta (including 0 and 1), padded
leading dimensions, a base pointer offset by 0 .. 3 floats (so 16-byte and
4-byte loads both occur), and a batch of 1 .. 3 with gaps between the
products; the result must meet the oracle's tolerance in every product, and
padding and gaps must be left untouched.  The small cases (sizes 1 .. 600)
mostly run the 16 x 16 small-product kernel, with some 32 x 32 and 32 x 64
tiles; the large cases run every buffer-to-LDS configuration but the 256 x
256 one (which the 8192^3 tests of every layout cover), four times each.  The
small cases also run through the bfloat16 split entry point (one product
each).
"""
import numpy as np
import pytest

import dense_fp32_matrix_03_amd as sg
import oracle
from dense_fp32_matrix_03_amd import inputs

pytestmark = pytest.mark.gpu

CASES = 400
LARGE_CASES = 40


@pytest.fixture(scope="module", autouse=True)
def library():
    sg.sgemm_create()
    yield
    sg.sgemm_destroy()


SMALL_DIMS = [1, 2, 3, 5, 16, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 200, 255, 256, 257,
              300, 384, 511, 600]
# (M, N, K, batch) of the large cases, one per buffer-to-LDS configuration
# on 256 CUs, in turn; layout, alpha, beta, padding and offset are drawn.
LARGE_SHAPES = [(1000, 1500, 777, 1),    # 64 x 96
                (512, 768, 515, 4),      # 64 x 96, a batch filling one round
                (2048, 2048, 256, 1),    # 128 x 128
                (1024, 1024, 1024, 1),   # 64 x 64 in two k sets
                (1024, 1024, 2048, 1),   # 64 x 64 in two k sets, 64-float slices
                (2048, 1536, 100, 1),    # 64 x 64, four waves, three rounds
                (800, 1280, 777, 1),     # 32 x 64
                (640, 640, 1024, 1),     # 32 x 64 with 64-float slices
                (768, 768, 777, 1),      # 32 x 32
                (512, 500, 515, 1)]      # 32 x 32 with 64-float slices


def _case(seed, large=False):
    g = np.random.default_rng(seed)
    if large:
        M, N, K, batch = LARGE_SHAPES[seed % len(LARGE_SHAPES)]
    else:
        M, N, K = (int(x) for x in g.choice(SMALL_DIMS, 3))
    ta, tb = bool(g.integers(0, 2)), bool(g.integers(0, 2))
    alpha = float(g.choice([1.0, -1.0, 0.5, 2.0, 0.0]))
    beta = float(g.choice([0.0, 1.0, -0.75, 0.0]))
    pad_a, pad_b, pad_c = (int(x) for x in g.integers(0, 5, 3))
    offset = int(g.integers(0, 4))
    if not large:
        batch = int(g.integers(1, 4))
    return g, M, N, K, ta, tb, alpha, beta, pad_a, pad_b, pad_c, offset, batch


def _layout(ta, tb, M, N, K, pad_a, pad_b):
    ar, ac = (K, M) if ta else (M, K)
    br, bc = (N, K) if tb else (K, N)
    return ar, ac, ac + pad_a, br, bc, bc + pad_b


@pytest.mark.parametrize("seed", range(CASES))
def test_general_form_random_case(seed):
    _general_case(10_000 + seed, False)


@pytest.mark.parametrize("seed", range(LARGE_CASES))
def test_general_form_random_large_case(seed):
    _general_case(30_000 + seed, True)


def _general_case(seed, large):
    import torch
    g, M, N, K, ta, tb, alpha, beta, pad_a, pad_b, pad_c, offset, batch = _case(seed, large)
    ar, ac, lda, br, bc, ldb = _layout(ta, tb, M, N, K, pad_a, pad_b)
    ldc = N + pad_c
    sA, sB, sC = ar * lda + 7, br * ldb + 5, M * ldc + 3
    As = [inputs.padded(inputs.uniform(g, (ar, ac)), lda) for _ in range(batch)]
    Bs = [inputs.padded(inputs.uniform(g, (br, bc)), ldb) for _ in range(batch)]
    C0s = [inputs.padded(inputs.uniform(g, (M, N)), ldc) for _ in range(batch)]
    bufA = np.full(offset + sA * batch, np.nan, np.float32)
    bufB = np.full(offset + sB * batch, np.nan, np.float32)
    bufC = np.full(offset + sC * batch, np.nan, np.float32)
    for b in range(batch):
        bufA[offset + b * sA:offset + b * sA + ar * lda] = As[b].ravel()
        bufB[offset + b * sB:offset + b * sB + br * ldb] = Bs[b].ravel()
        bufC[offset + b * sC:offset + b * sC + M * ldc] = C0s[b].ravel()
    dA = torch.from_numpy(bufA).cuda()
    dB = torch.from_numpy(bufB).cuda()
    dC = torch.from_numpy(bufC).cuda()
    shift = 4 * offset
    print(f"case {seed}: {'T' if ta else 'N'}{'T' if tb else 'N'} M={M} N={N} K={K} "
          f"alpha={alpha} beta={beta} lds=({lda},{ldb},{ldc}) offset={offset} batch={batch}",
          flush=True)
    sg.sgemm_run_strided_batched(ta, tb, M, N, K, alpha, dA.data_ptr() + shift, lda, sA,
                                 dB.data_ptr() + shift, ldb, sB, beta, dC.data_ptr() + shift,
                                 ldc, sC, batch)
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    assert np.all(np.isnan(out[:offset]))
    for b in range(batch):
        C = out[offset + b * sC:offset + b * sC + M * ldc].reshape(M, ldc)
        Cref, Sabs = oracle.sgemm_ex_f64(ta, tb, M, N, K, alpha, As[b], Bs[b], beta, C0s[b])
        r = oracle.check(C[:, :N], Cref, Sabs)
        assert r.ok, f"case {seed} product {b}: {r}"
        assert np.array_equal(C[:, N:].view(np.uint32), C0s[b][:, N:].view(np.uint32)), \
            "padding columns of C changed"
        gap = out[offset + b * sC + M * ldc:offset + (b + 1) * sC]
        assert np.all(np.isnan(gap)), "gap after a product changed"


@pytest.mark.parametrize("seed", range(0, CASES, 3))
def test_bf16x3_random_case(seed):
    import torch
    g, M, N, K, ta, tb, alpha, beta, pad_a, pad_b, pad_c, offset, _ = _case(20_000 + seed)
    ar, ac, lda, br, bc, ldb = _layout(ta, tb, M, N, K, pad_a, pad_b)
    ldc = N + pad_c
    A = inputs.padded(inputs.uniform(g, (ar, ac)), lda)
    B = inputs.padded(inputs.uniform(g, (br, bc)), ldb)
    C0 = inputs.padded(inputs.uniform(g, (M, N)), ldc)
    dA = torch.from_numpy(np.concatenate([np.full(offset, np.nan, np.float32), A.ravel()])).cuda()
    dB = torch.from_numpy(np.concatenate([np.full(offset, np.nan, np.float32), B.ravel()])).cuda()
    dC = torch.from_numpy(C0.copy()).cuda()
    nbytes = sg.sgemm_bf16x3_workspace_size(M, N, K)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    shift = 4 * offset
    print(f"bf16x3 case {seed}: {'T' if ta else 'N'}{'T' if tb else 'N'} M={M} N={N} K={K} "
          f"alpha={alpha} beta={beta} offset={offset}", flush=True)
    sg.sgemm_run_bf16x3_ex(ta, tb, M, N, K, alpha, dA.data_ptr() + shift, lda,
                           dB.data_ptr() + shift, ldb, beta, dC, ldc, ws, nbytes)
    torch.cuda.synchronize()
    C = dC.cpu().numpy()
    Cref, Sabs = oracle.sgemm_ex_f64(ta, tb, M, N, K, alpha, A, B, beta, C0)
    r = oracle.check(C[:, :N], Cref, Sabs)
    assert r.ok, f"bf16x3 case {seed}: {r}"
    assert np.array_equal(C[:, N:].view(np.uint32), C0[:, N:].view(np.uint32))
