"""The entry points under HIP graph capture: each call launches kernels only
(no allocation, no memset), so a captured graph replays them.  Every replay
is checked against the eager result, with eager work and synchronisation
between replays."""
import numpy as np
import pytest

import dense_fp32_matrix_03_amd as sg
from dense_fp32_matrix_03_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def library():
    sg.sgemm_create()
    yield
    sg.sgemm_destroy()


def _replays_match(capture_body, out, eager_bits, replays=5):
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        capture_body()  # warm-up on the side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        capture_body()
    for r in range(replays):
        out.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert out.cpu().numpy().tobytes() == eager_bits, f"replay {r}"


# 520 x 384 x 260 runs the buffer-to-LDS kernel (32 x 32 tile, four k sets);
# 256 x 256 x 256 the 16 x 16 small-product kernel.
@pytest.mark.parametrize("M,N,K", [(520, 384, 260), (256, 256, 256)])
def test_sgemm_run_and_general_form_in_a_graph(M, N, K):
    import torch
    g0 = np.random.default_rng(61 + M)
    dA = torch.from_numpy(inputs.uniform(g0, (M, K))).cuda()
    dBt = torch.from_numpy(inputs.uniform(g0, (N, K))).cuda()
    dB = dBt.t().contiguous()
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    C2 = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def body():
        sg.sgemm_run(M, N, K, dA, K, dB, N, C, N)
        sg.sgemm_run_ex(0, 1, M, N, K, -0.5, dA, K, dBt, K, 0.0, C2, N)

    body()
    torch.cuda.synchronize()
    eager, eager2 = C.cpu().numpy().tobytes(), C2.cpu().numpy().tobytes()
    _replays_match(body, C, eager)
    assert C2.cpu().numpy().tobytes() == eager2


def test_bf16x3_and_vector_add_in_a_graph():
    import torch
    g0 = np.random.default_rng(67)
    M, N, K = 300, 200, 100
    dA = torch.from_numpy(inputs.uniform(g0, (M, K))).cuda()
    dB = torch.from_numpy(inputs.uniform(g0, (K, N))).cuda()
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nbytes = sg.sgemm_bf16x3_workspace_size(M, N, K)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    va, vb = inputs.vector_add_inputs(100_001, "uniform", seed=3)
    dva, dvb = torch.from_numpy(va).cuda(), torch.from_numpy(vb).cuda()
    dvc = torch.empty_like(dva)

    def body():
        sg.sgemm_run_bf16x3(M, N, K, dA, K, dB, N, C, N, ws, nbytes)
        sg.vector_add(100_001, dva, dvb, dvc)

    body()
    torch.cuda.synchronize()
    eager, eager_v = C.cpu().numpy().tobytes(), dvc.cpu().numpy().tobytes()
    _replays_match(body, C, eager)
    assert dvc.cpu().numpy().tobytes() == eager_v
