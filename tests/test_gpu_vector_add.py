"""Vector addition on the GPU (vector_add in include/vector_add.h) against the
oracle: bit-exact, since both sides round each single sum to nearest even."""
import numpy as np
import pytest

import dense_fp32_matrix_03_amd as sg
import oracle
from dense_fp32_matrix_03_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def library():
    sg.sgemm_create()
    yield
    sg.sgemm_destroy()


def _run(A, B, offset=(0, 0, 0)):
    """Run on device copies placed `offset` floats into their buffers."""
    import torch
    n = A.shape[0]
    oa, ob, oc = offset
    dA = torch.full((n + oa + 8,), float("nan"), dtype=torch.float32, device="cuda")
    dB = torch.full((n + ob + 8,), float("nan"), dtype=torch.float32, device="cuda")
    dC = torch.full((n + oc + 8,), float("nan"), dtype=torch.float32, device="cuda")
    dA[oa:oa + n] = torch.from_numpy(A).cuda()
    dB[ob:ob + n] = torch.from_numpy(B).cuda()
    sg.vector_add(n, dA[oa:], dB[ob:], dC[oc:])
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    assert np.all(np.isnan(out[:oc])) and np.all(np.isnan(out[oc + n:])), "wrote outside C"
    return out[oc:oc + n]


def _same_bits(x, y):
    return np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_sin_cos_full_size():
    """The blog's experiment: n = 2^24, A = sin^2(i), B = cos^2(i)."""
    A, B = inputs.vector_add_inputs()
    C = _run(A, B)
    assert _same_bits(C, oracle.vector_add(A, B))
    assert float(np.max(np.abs(C.astype(np.float64) - 1.0))) <= 8 * 2.0 ** -24


@pytest.mark.parametrize("n", [1, 3, 4, 5, 255, 1023, 1024, 1025, 4097, 1_000_003])
def test_ragged_lengths(n):
    A, B = inputs.vector_add_inputs(n, "uniform", seed=n)
    assert _same_bits(_run(A, B), oracle.vector_add(A, B))


@pytest.mark.parametrize("offset", [(1, 0, 0), (0, 2, 0), (0, 0, 3), (1, 1, 1), (4, 8, 12)])
def test_unaligned_operands(offset):
    A, B = inputs.vector_add_inputs(100_003, "uniform", seed=7)
    assert _same_bits(_run(A, B, offset), oracle.vector_add(A, B))


def test_special_values():
    big = np.finfo(np.float32).max
    tiny = np.uint32(1).view(np.float32)
    A = np.float32([2.5, -7.0, 0.0, big, np.nan, -0.0, tiny, 1.0, 1.0 + 2.0 ** -23])
    B = np.float32([-2.5, 0.0, -0.0, big, 1.0, -0.0, tiny, 2.0 ** -24, 2.0 ** -24])
    C = _run(A, B)
    ref = oracle.vector_add(A, B)
    assert _same_bits(C[~np.isnan(ref)], ref[~np.isnan(ref)])
    assert np.isnan(C[4])


def test_in_place():
    import torch
    A, B = inputs.vector_add_inputs(50_000, "uniform", seed=9)
    dA = torch.from_numpy(A).cuda()
    dB = torch.from_numpy(B).cuda()
    sg.vector_add(A.shape[0], dA, dB, dA)
    torch.cuda.synchronize()
    assert _same_bits(dA.cpu().numpy(), oracle.vector_add(A, B))


def test_zero_length_and_errors():
    import torch
    d = torch.zeros(4, device="cuda")
    sg.vector_add(0, d, d, d)
    with pytest.raises(sg.SgemmError):
        sg.vector_add(-1, d, d, d)
    with pytest.raises(sg.SgemmError):
        sg.vector_add(4, d, None, d)
