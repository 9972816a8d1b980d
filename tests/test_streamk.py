"""GPU parity of the stream-K configuration (d256x256x32_s4_isk) against the oracle.

Stream-K splits the K steps of the tiles that do not fill a whole round of CUs
into near-equal ranges, one per workgroup; the pieces of a tile publish fp32
partials and the last to arrive stores the tile from their sum, in piece order.
These cases force the configuration and the number of stream-K workgroups
(GEMM_RELU_SK_UNITS) so that tiles are split into 1, 2, 3 and many pieces,
pieces end inside the K tail, whole-tile workgroups precede the split ones, and
every workgroup takes a single K step.  Integer-valued inputs have one correct
result in any summation order (bit-exact); random inputs are held to the fp32
summation bound and must repeat bit for bit from call to call (the sum order is
fixed, whichever piece arrives last).
"""
import numpy as np
import pytest

import dense_tiled_gemm_relu_amd as gr
import oracle
import workloads as wl
from tests.helpers import (built_configs, check_close, from_device, fp32_sum_bound, out_tensor,
                           to_device, unit_roundoff)

SK = "d256x256x32_s4_isk"

# a comparison configuration: in the library only when it is built with
# GEMM_RELU_COMPARISON_CONFIGS=1
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not built_configs([SK]),
                                 reason="stream-K is a comparison configuration, not in this build")]


@pytest.fixture(autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    yield


def upload(A, B, M, N, K, in_code, out_code, transB):
    Ad, Bd = to_device(A, in_code, (M, K)), to_device(B, in_code, wl.b_shape(M, N, K, transB))
    return Ad, Bd, out_tensor(M, N, out_code, float("nan"))


def run_sk(A, B, M, N, K, in_code, out_code, transB, units, monkeypatch, stream=None):
    import torch
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", SK)
    monkeypatch.setenv("GEMM_RELU_SK_UNITS", str(units))
    Ad, Bd, Cd = upload(A, B, M, N, K, in_code, out_code, transB)
    assert gr.gemm_relu_plan(Ad, Bd, Cd, M, N, K, in_code, out_code, transB) == SK
    gr.gemm_relu(Ad, Bd, Cd, M, N, K, in_code, out_code, transB, stream)
    torch.cuda.synchronize()
    return from_device(Cd)


def int_inputs(M, N, K, in_code, transB, seed, out_code):
    lo, hi = (-1, 1) if out_code == wl.BF16 else (-2, 2)
    A = wl.integers((M, K), seed, in_code, lo, hi)
    B = wl.integers(wl.b_shape(M, N, K, transB), seed + 1, in_code, lo, hi)
    return A, B


# (M, N, K): 2x3 tiles of 7 K steps (the last one a 8-wide tail); ragged 2x3
# tiles of 7 steps; 3x2 tiles of 32 steps with a tail of 8
SHAPES = [(264, 520, 200), (301, 517, 203), (513, 300, 1000)]
# units: 0 = one workgroup per CU (the default); 1 = one workgroup walks every tile; 5, 13:
# 2 to 4 pieces a tile, pieces starting and ending mid-tile; 42: one K step
# per workgroup on the 7-step shapes (7 pieces a tile, the last ones in the tail)
UNITS = [0, 1, 5, 13, 42]


@pytest.mark.parametrize("units", UNITS)
@pytest.mark.parametrize("shape", SHAPES, ids=["k7", "ragged", "k32"])
@pytest.mark.parametrize("in_code,out_code", [(wl.F16, wl.F16), (wl.BF16, wl.F32), (wl.F16, wl.BF16)])
@pytest.mark.parametrize("transB", [0, 1])
def test_streamk_integer_bitexact(units, shape, in_code, out_code, transB, monkeypatch):
    M, N, K = shape
    A, B = int_inputs(M, N, K, in_code, transB, 300, out_code)
    ref = oracle.gemm_relu_ref(A, B, M, N, K, in_code, transB)
    got = run_sk(A, B, M, N, K, in_code, out_code, transB, units, monkeypatch)
    assert np.array_equal(got, ref)
    assert not np.any(np.signbit(got))


@pytest.mark.parametrize("units", [0, 37, 112])
@pytest.mark.parametrize("transB", [0, 1])
def test_streamk_after_whole_tile_round(units, transB, monkeypatch):
    """17 x 16 = 272 tiles: 256 whole-tile workgroups, then the remaining 16
    tiles' 7 K steps each over the stream-K workgroups."""
    M, N, K = 4352, 4096, 200
    A, B = int_inputs(M, N, K, wl.F16, transB, 310, wl.F16)
    ref = oracle.gemm_relu_ref(A, B, M, N, K, wl.F16, transB)
    got = run_sk(A, B, M, N, K, wl.F16, wl.F16, transB, units, monkeypatch)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("units", [0, 13, 42])
@pytest.mark.parametrize("in_code", [wl.F8E4M3, wl.F8E5M2])
@pytest.mark.parametrize("transB", [0, 1])
def test_streamk_fp8_integer_bitexact(units, in_code, transB, monkeypatch):
    # 8-bit inputs take 64 elements a K step: 2x3 tiles of 7 steps, a tail of 8
    M, N, K = 301, 517, 392
    A = wl.integers((M, K), 320, in_code, -2, 2)
    B = wl.integers(wl.b_shape(M, N, K, transB), 321, in_code, -2, 2)
    ref = oracle.gemm_relu_ref(A, B, M, N, K, in_code, transB)
    got = run_sk(A, B, M, N, K, in_code, wl.F16, transB, units, monkeypatch)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("units", [0, 5, 13, 42])
@pytest.mark.parametrize("in_code,out_code", [(wl.F16, wl.F16), (wl.BF16, wl.F32)])
def test_streamk_uniform_tolerance_and_repeatable(units, in_code, out_code, monkeypatch):
    import torch
    M, N, K = 301, 517, 203
    A, B = wl.make_inputs(M, N, K, in_code, 0, "uniform", 330)
    ref = oracle.gemm_relu_ref(A, B, M, N, K, in_code, 0)
    first = run_sk(A, B, M, N, K, in_code, out_code, 0, units, monkeypatch)
    check_close(first, ref, K, out_code)
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    _, absum = oracle.gemm_relu_ref_at(A, B, rows.ravel(), cols.ravel(), M, N, K, in_code, 0)
    bound = fp32_sum_bound(absum.reshape(M, N), ref, K, unit_roundoff(out_code))
    assert np.all(np.abs(first - ref) <= bound)
    # the arrival counters return to zero, and the sum order does not depend
    # on which piece arrives last: further calls repeat the first bit for bit
    Ad, Bd, Cd = upload(A, B, M, N, K, in_code, out_code, 0)
    for _ in range(4):
        Cd.fill_(float("nan"))
        gr.gemm_relu(Ad, Bd, Cd, M, N, K, in_code, out_code, 0)
        torch.cuda.synchronize()
        assert np.array_equal(from_device(Cd), first)


def test_streamk_two_streams(monkeypatch):
    """Calls on two streams at once use separate workspaces."""
    import torch
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", SK)
    monkeypatch.setenv("GEMM_RELU_SK_UNITS", "13")
    M, N, K = 513, 300, 1000
    cases = []
    for seed in (340, 342):
        A, B = int_inputs(M, N, K, wl.F16, 1, seed, wl.F16)
        cases.append((oracle.gemm_relu_ref(A, B, M, N, K, wl.F16, 1),
                      upload(A, B, M, N, K, wl.F16, wl.F16, 1)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for _ in range(3):
        for (ref, (Ad, Bd, Cd)), s in zip(cases, streams):
            gr.gemm_relu(Ad, Bd, Cd, M, N, K, wl.F16, wl.F16, 1, s)
    torch.cuda.synchronize()
    for ref, (_, _, Cd) in cases:
        assert np.array_equal(from_device(Cd), ref)


def test_streamk_graph_capture(monkeypatch):
    """Under capture the call takes whole tiles (nothing is allocated, and no
    per-stream workspace is shared with the graph), also once an eager call on
    that stream has set one up; the captured launch replays correctly, eager
    stream-K calls in between."""
    import torch
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", SK)
    monkeypatch.setenv("GEMM_RELU_SK_UNITS", "13")
    M, N, K = 513, 300, 1000
    A, B = int_inputs(M, N, K, wl.F16, 0, 350, wl.F16)
    ref = oracle.gemm_relu_ref(A, B, M, N, K, wl.F16, 0)
    A2, B2 = int_inputs(M, N, K, wl.F16, 0, 352, wl.F16)
    ref2 = oracle.gemm_relu_ref(A2, B2, M, N, K, wl.F16, 0)
    Ad, Bd, Cd = upload(A, B, M, N, K, wl.F16, wl.F16, 0)
    A2d, B2d, C2d = upload(A2, B2, M, N, K, wl.F16, wl.F16, 0)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    for warm in (False, True):
        if warm:
            with torch.cuda.stream(s):
                gr.gemm_relu(Ad, Bd, Cd, M, N, K, wl.F16, wl.F16, 0, s)
            s.synchronize()
            assert np.array_equal(from_device(Cd), ref)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            gr.gemm_relu(Ad, Bd, Cd, M, N, K, wl.F16, wl.F16, 0, s)
        for _ in range(3):
            Cd.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(from_device(Cd), ref)
            with torch.cuda.stream(s):
                C2d.fill_(float("nan"))
                gr.gemm_relu(A2d, B2d, C2d, M, N, K, wl.F16, wl.F16, 0, s)
            s.synchronize()
            assert np.array_equal(from_device(C2d), ref2)
        del g
