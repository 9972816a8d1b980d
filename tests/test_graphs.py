"""The C-ABI entry points under HIP graph capture.

gemm_relu and gemm_relu_ws allocate nothing and clear nothing with memset
nodes (the K split's arrival counters return to zero inside the kernel), so a
call may be captured into a graph and replayed.  Each case captures one call,
then replays the graph several times with the program's own eager work (other
calls on the same stream and workspace, fills of the output) in between, and
checks every replay bit for bit against the oracle on integer inputs.  The
no-allocation entry point's capture is tested with it, in the file that runs
last.
"""
import numpy as np
import pytest

import dense_tiled_gemm_relu_amd as gr
import oracle
import workloads as wl
from tests.helpers import from_device, out_tensor, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    yield


def int_inputs(M, N, K, transB, seed):
    A = wl.integers((M, K), seed, wl.F16, -2, 2)
    B = wl.integers(wl.b_shape(M, N, K, transB), seed + 1, wl.F16, -2, 2)
    return A, B


# a ragged shape on a smaller tile, the eight-wave 256x256 tile, and the
# two-region grid
CASES = [(300, 520, 264, 0, None), (4096, 4096, 512, 0, "d256x256x32_s4_i16w8"),
         (4096, 7168, 256, 1, "d256x256x32_s4_i16+d256x192x32_s4_i16")]


@pytest.mark.parametrize("M,N,K,transB,plan", CASES)
def test_gemm_relu_captured_and_replayed(M, N, K, transB, plan):
    import torch
    A, B = int_inputs(M, N, K, transB, 1200 + M)
    ref = oracle.gemm_relu_ref_matmul(A, B, M, N, K, wl.F16, transB)
    A2, B2 = int_inputs(M, N, K, transB, 1300 + M)
    ref2 = oracle.gemm_relu_ref_matmul(A2, B2, M, N, K, wl.F16, transB)
    Ad, Bd = to_device(A, wl.F16, (M, K)), to_device(B, wl.F16, wl.b_shape(M, N, K, transB))
    A2d, B2d = to_device(A2, wl.F16, (M, K)), to_device(B2, wl.F16, wl.b_shape(M, N, K, transB))
    Cd, C2d = out_tensor(M, N, wl.F16, float("nan")), out_tensor(M, N, wl.F16, float("nan"))
    if plan is not None:
        assert gr.gemm_relu_plan(Ad, Bd, Cd, M, N, K, wl.F16, wl.F16, transB) == plan
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):          # an eager call first, as a program would
        gr.gemm_relu(Ad, Bd, Cd, M, N, K, wl.F16, wl.F16, transB, s)
    s.synchronize()
    assert np.array_equal(from_device(Cd), ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        gr.gemm_relu(Ad, Bd, Cd, M, N, K, wl.F16, wl.F16, transB, s)
    for _ in range(3):
        Cd.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(from_device(Cd), ref)
        with torch.cuda.stream(s):
            C2d.fill_(float("nan"))
            gr.gemm_relu(A2d, B2d, C2d, M, N, K, wl.F16, wl.F16, transB, s)
        s.synchronize()
        assert np.array_equal(from_device(C2d), ref2)
    del g


@pytest.mark.parametrize("transB", [0, 1])
def test_gemm_relu_ws_split_captured_and_replayed(transB):
    """The K split on a caller's workspace: the graph's launch and eager calls
    share the workspace on one stream; each replay must find the arrival
    counters as the previous call left them (zero)."""
    import torch
    M, N, K = 64, 2048, 8192
    A, B = int_inputs(M, N, K, transB, 1400)
    ref = oracle.gemm_relu_ref_matmul(A, B, M, N, K, wl.F16, transB)
    A2, B2 = int_inputs(M, N, K, transB, 1500)
    ref2 = oracle.gemm_relu_ref_matmul(A2, B2, M, N, K, wl.F16, transB)
    Ad, Bd = to_device(A, wl.F16, (M, K)), to_device(B, wl.F16, wl.b_shape(M, N, K, transB))
    A2d, B2d = to_device(A2, wl.F16, (M, K)), to_device(B2, wl.F16, wl.b_shape(M, N, K, transB))
    Cd, C2d = out_tensor(M, N, wl.F16, float("nan")), out_tensor(M, N, wl.F16, float("nan"))
    need = gr.gemm_relu_workspace_size(M, N, K, wl.F16, wl.F16, transB)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    assert gr.gemm_relu_ws_plan(Ad, Bd, Cd, M, N, K, wl.F16, wl.F16, transB, ws, need).endswith("_splitk")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        gr.gemm_relu_ws(Ad, Bd, Cd, M, N, K, wl.F16, wl.F16, transB, ws, need, s)
    s.synchronize()
    assert np.array_equal(from_device(Cd), ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        gr.gemm_relu_ws(Ad, Bd, Cd, M, N, K, wl.F16, wl.F16, transB, ws, need, s)
    for _ in range(4):
        with torch.cuda.stream(s):          # replays and eager calls ordered on one stream
            Cd.fill_(float("nan"))
            g.replay()
            C2d.fill_(float("nan"))
            gr.gemm_relu_ws(A2d, B2d, C2d, M, N, K, wl.F16, wl.F16, transB, ws, need, s)
        s.synchronize()
        assert np.array_equal(from_device(Cd), ref)
        assert np.array_equal(from_device(C2d), ref2)
    assert bool((ws[:4096] == 0).all())
    del g
