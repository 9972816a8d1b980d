"""gemm_relu_noalloc: the K split of gemm_relu_ws with the library's own per-GPU
scratch array as the workspace, for callers that cannot allocate.

Its output must be that of gemm_relu_ws with a caller's workspace bit for bit
(the same kernels, parts and summation order), call after call on the shared
array, including a smaller problem after a larger one.
"""
import numpy as np
import pytest

import dense_tiled_gemm_relu_amd as gr
import workloads as wl
from tests.helpers import from_device, out_tensor, to_device

SPLITK = "d64x128x64_s4_splitk"
FAKE = 1 << 40


def test_rejects_a_split_beyond_the_scratch(monkeypatch):
    """A forced split of 1024 tiles in 16 parts needs 512 MiB: refused before
    any device work, with its own status and message."""
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", SPLITK)
    monkeypatch.setenv("GEMM_RELU_SPLITK_PARTS", "16")
    M, N, K = 2048, 4096, 4096
    assert gr.gemm_relu_workspace_size(M, N, K, wl.F16, wl.F16, 0) > 16 << 20
    a, b = FAKE, FAKE + (1 << 32)
    c = b + (1 << 32)
    assert gr.gemm_relu_noalloc_status(a, b, c, M, N, K, wl.F16, wl.F16, 0, 0) == gr.ESCRATCH
    assert "scratch" in gr.gemm_relu_strerror(gr.ESCRATCH)


def test_invalid_arguments_as_gemm_relu():
    assert gr.gemm_relu_noalloc_status(FAKE, FAKE + 4096, FAKE, 64, 64, 64, wl.F16, wl.F16, 0,
                                       0) == gr.EINVAL     # C over A
    assert gr.gemm_relu_noalloc_status(0, 0, FAKE, 64, 64, 64, wl.F16, wl.F16, 0, 0) == gr.EINVAL
    assert gr.gemm_relu_noalloc_status(FAKE, FAKE, FAKE, 0, 64, 64, wl.F16, wl.F16, 0, 0) == gr.OK


def _pair(M, N, K, transB, seed):
    """gemm_relu_noalloc and gemm_relu_ws (a zeroed caller workspace) on the
    same uniform inputs; returns both outputs and the ws plan."""
    import torch
    A = wl.uniform((M, K), seed, wl.F16)
    B = wl.uniform(wl.b_shape(M, N, K, transB), seed + 1, wl.F16)
    Ad, Bd = to_device(A, wl.F16, (M, K)), to_device(B, wl.F16, wl.b_shape(M, N, K, transB))
    need = gr.gemm_relu_workspace_size(M, N, K, wl.F16, wl.F16, transB)
    ws = torch.zeros(max(need, 4096), dtype=torch.uint8, device="cuda")
    C_ws = out_tensor(M, N, wl.F16, float("nan"))
    C_na = out_tensor(M, N, wl.F16, float("nan"))
    plan = gr.gemm_relu_ws_plan(Ad, Bd, C_ws, M, N, K, wl.F16, wl.F16, transB, ws, need)
    gr.gemm_relu_ws(Ad, Bd, C_ws, M, N, K, wl.F16, wl.F16, transB, ws, need)
    gr.gemm_relu_noalloc(Ad, Bd, C_na, M, N, K, wl.F16, wl.F16, transB)
    torch.cuda.synchronize()
    return from_device(C_na), from_device(C_ws), plan


@pytest.mark.gpu
def test_matches_the_workspace_entry_two_calls_in_a_row():
    """The skinny 64 x 8192 x 8192 product, then a smaller one (fewer tiles,
    more parts) on the same scratch: each bit for bit as gemm_relu_ws."""
    got, want, plan = _pair(64, 8192, 8192, 0, 800)
    assert plan == SPLITK
    assert not np.any(np.isnan(got))
    assert np.array_equal(got, want)
    got, want, plan = _pair(40, 2048, 4096, 0, 810)
    assert plan == SPLITK
    assert np.array_equal(got, want)


@pytest.mark.gpu
def test_matches_where_nothing_splits():
    """A shape the plan does not split runs as gemm_relu, scratch untouched."""
    got, want, plan = _pair(300, 260, 520, 1, 820)
    assert plan != SPLITK
    assert np.array_equal(got, want)


@pytest.mark.gpu
def test_captured_and_replayed():
    """Captured into a graph (after an eager call has looked up the scratch's
    address on this GPU) and replayed, with eager calls of another shape on
    the same scratch and stream in between: every result as gemm_relu_ws's."""
    import torch
    M, N, K = 64, 4096, 8192
    A = wl.uniform((M, K), 830, wl.F16)
    B = wl.uniform((K, N), 831, wl.F16)
    Ad, Bd = to_device(A, wl.F16, (M, K)), to_device(B, wl.F16, (K, N))
    want, _, plan = _pair(M, N, K, 0, 830)
    assert plan == SPLITK
    M2, N2, K2 = 40, 2048, 4096
    want2, _, _ = _pair(M2, N2, K2, 0, 840)
    A2 = wl.uniform((M2, K2), 840, wl.F16)
    B2 = wl.uniform((K2, N2), 841, wl.F16)
    A2d, B2d = to_device(A2, wl.F16, (M2, K2)), to_device(B2, wl.F16, (K2, N2))
    Cd, C2d = out_tensor(M, N, wl.F16, float("nan")), out_tensor(M2, N2, wl.F16, float("nan"))
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        gr.gemm_relu_noalloc(Ad, Bd, Cd, M, N, K, wl.F16, wl.F16, 0, s)
    for _ in range(3):
        with torch.cuda.stream(s):
            Cd.fill_(float("nan"))
            g.replay()
            C2d.fill_(float("nan"))
            gr.gemm_relu_noalloc(A2d, B2d, C2d, M2, N2, K2, wl.F16, wl.F16, 0, s)
        s.synchronize()
        assert np.array_equal(from_device(Cd), want)
        assert np.array_equal(from_device(C2d), want2)
    del g
