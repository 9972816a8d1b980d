"""gemm_relu_ws with stream-K on the eight-wave 256x256 tile
(d256x256x32_s4_i16w8sk, a comparison configuration) against the oracle.

Where the 256x256 tiles leave the last round of CUs partly empty, whole rounds
keep one workgroup per tile and the remaining tiles' K steps are shared out in
near-equal ranges, one per workgroup (the T.Persistent / stream-K idea of page
"TileLang：GPU/NPU 通用算子 DSL", §3.3).  The pieces of a tile publish fp32
partials in the caller's workspace; the last to arrive adds them in piece
order and applies the ReLU once, to the whole sum.  So the bars are
gemm_relu's: bit for bit on integer inputs, the contract and fp32-summation
bounds on random ones, and the same bits from call to call (the sum order is
fixed, whichever piece arrives last).  GEMM_RELU_SK_UNITS forces the number of
stream-K workgroups so that tiles are split into 1, 2, 3 and many pieces,
pieces end inside the K tail, and a workgroup walks several tiles.  Plan
selection never takes it (it is slower than whole tiles); only
GEMM_RELU_FORCE_CONFIG does, in a library built with the comparison
configurations.
"""
import numpy as np
import pytest

import dense_tiled_gemm_relu_amd as gr
import oracle
import workloads as wl
from tests.helpers import (built_configs, check_close, from_device, fp32_sum_bound, out_tensor,
                           to_device, unit_roundoff)

SK = "d256x256x32_s4_i16w8sk"
FLAG_BYTES = 4096          # arrival counters, before the partial tiles
SLOT = 256 * 256 * 4       # one fp32 partial tile
FAKE = 1 << 40
need_sk = pytest.mark.skipif(not built_configs([SK]),
                             reason="stream-K is a comparison configuration, not in this build")


def need_bytes(units):
    return FLAG_BYTES + 2 * units * SLOT


def fake_args(M, N, K, eb=2):
    a = FAKE
    b = a + M * K * eb + 4096
    c = b + K * N * eb + 4096
    w = ((c + M * N * 4 + 4096) + 255) // 256 * 256
    return a, b, c, w


# ------------------------------------------------------------ host side
@pytest.mark.parametrize("M,N,K,ic,oc,tb", [(4096, 7168, 4096, wl.BF16, wl.F32, 1),
                                            (4097, 3001, 5003, wl.F16, wl.F16, 0)])
def test_plan_selection_never_takes_it(M, N, K, ic, oc, tb):
    a, b, c, w = fake_args(M, N, K)
    assert gr.gemm_relu_workspace_size(M, N, K, ic, oc, tb) == 0
    assert gr.gemm_relu_ws_plan(a, b, c, M, N, K, ic, oc, tb, w, need_bytes(256)) == \
        gr.gemm_relu_plan(a, b, c, M, N, K, ic, oc, tb)


@need_sk
def test_forced_workspace_sizes(monkeypatch):
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", SK)
    # bf16 4096 x 7168 x 4096: 448 tiles = 256 whole + 192 split over 256 units
    assert gr.gemm_relu_workspace_size(4096, 7168, 4096, wl.BF16, wl.F32, 1) == need_bytes(256)
    # 4097 x 3001 x 5003: 204 tiles, all split (0.8 of a round)
    assert gr.gemm_relu_workspace_size(4097, 3001, 5003, wl.F16, wl.F16, 0) == need_bytes(256)
    # whole rounds, 8-bit inputs: none
    assert gr.gemm_relu_workspace_size(8192, 8192, 8192, wl.F16, wl.F16, 0) == 0
    assert gr.gemm_relu_workspace_size(4096, 7168, 4096, wl.F8E4M3, wl.F16, 0) == 0
    monkeypatch.setenv("GEMM_RELU_SK_UNITS", "5")
    assert gr.gemm_relu_workspace_size(300, 500, 64, wl.F16, wl.F16, 0) == need_bytes(5)
    a, b, c, w = fake_args(300, 500, 64)
    assert gr.gemm_relu_ws_plan(a, b, c, 300, 500, 64, wl.F16, wl.F16, 0, w, need_bytes(5)) == SK
    # too small a workspace: the workspace-free plan
    assert gr.gemm_relu_ws_plan(a, b, c, 300, 500, 64, wl.F16, wl.F16, 0, w, need_bytes(5) - 1) != SK
    # gemm_relu itself never takes it
    assert gr.gemm_relu_plan(a, b, c, 300, 500, 64, wl.F16, wl.F16, 0) != SK


# ------------------------------------------------------------ GPU
def _ws(nbytes, fill=None):
    import torch
    t = torch.zeros(max(nbytes, FLAG_BYTES), dtype=torch.uint8, device="cuda")
    assert t.data_ptr() % 256 == 0
    if fill is not None and t.numel() > FLAG_BYTES:
        t[FLAG_BYTES:].view(torch.float32).fill_(fill)
    return t


def counters_zero(ws):
    return bool((ws[:FLAG_BYTES] == 0).all())


def run_ws(A, B, M, N, K, in_code, out_code, transB, ws_fill=None, expect=SK):
    import torch
    Ad, Bd = to_device(A, in_code, (M, K)), to_device(B, in_code, wl.b_shape(M, N, K, transB))
    Cd = out_tensor(M, N, out_code, float("nan"))
    need = gr.gemm_relu_workspace_size(M, N, K, in_code, out_code, transB)
    ws = _ws(need, ws_fill)
    assert gr.gemm_relu_ws_plan(Ad, Bd, Cd, M, N, K, in_code, out_code, transB, ws, ws.numel()) == expect
    gr.gemm_relu_ws(Ad, Bd, Cd, M, N, K, in_code, out_code, transB, ws, ws.numel())
    torch.cuda.synchronize()
    assert counters_zero(ws)
    return from_device(Cd)


def int_inputs(M, N, K, in_code, transB, seed, out_code):
    lo, hi = (-1, 1) if out_code == wl.BF16 else (-2, 2)
    return (wl.integers((M, K), seed, in_code, lo, hi),
            wl.integers(wl.b_shape(M, N, K, transB), seed + 1, in_code, lo, hi))


EXACT = {wl.F16: 2048.0, wl.BF16: 256.0, wl.F32: 2.0 ** 24}
# 2x3 tiles of 7 K steps (the last a tail of 8); ragged 2x3 tiles of 7 steps;
# 3x2 tiles of 32 steps and a tail of 8
SHAPES = [(264, 520, 200), (301, 517, 203), (513, 300, 1000)]
# 0: one unit per CU (single-step pieces here, many a tile); 1: one unit walks
# every tile; 5, 13: 2 to 4 pieces a tile, starting and ending mid-tile
UNITS = [0, 1, 5, 13]


@pytest.mark.gpu
@need_sk
@pytest.mark.parametrize("units", UNITS)
@pytest.mark.parametrize("shape", SHAPES, ids=["k7", "ragged", "k32"])
@pytest.mark.parametrize("in_code,out_code", [(wl.F16, wl.F16), (wl.BF16, wl.F32), (wl.F16, wl.BF16)])
@pytest.mark.parametrize("transB", [0, 1])
def test_forced_streamk_integer_bitexact(units, shape, in_code, out_code, transB, monkeypatch):
    M, N, K = shape
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", SK)
    monkeypatch.setenv("GEMM_RELU_SK_UNITS", str(units))
    A, B = int_inputs(M, N, K, in_code, transB, 800, out_code)
    ref = oracle.gemm_relu_ref_matmul(A, B, M, N, K, in_code, transB)
    assert np.abs(ref).max() < EXACT[out_code]
    got = run_ws(A, B, M, N, K, in_code, out_code, transB, ws_fill=float("nan"))
    assert np.array_equal(got, ref)
    assert not np.any(np.signbit(got))


@pytest.mark.gpu
@need_sk
@pytest.mark.parametrize("transB", [0, 1])
def test_forced_streamk_uniform_repeatable(transB, monkeypatch):
    """Random inputs within the bounds, the same bits on every call whatever
    the workspace held, and one workspace for back-to-back calls."""
    import torch
    M, N, K = 600, 700, 1500
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", SK)
    monkeypatch.setenv("GEMM_RELU_SK_UNITS", "7")
    A = wl.uniform((M, K), 810, wl.F16)
    B = wl.uniform(wl.b_shape(M, N, K, transB), 811, wl.F16)
    first = run_ws(A, B, M, N, K, wl.F16, wl.F16, transB, ws_fill=float("nan"))
    ref = oracle.gemm_relu_ref(A, B, M, N, K, wl.F16, transB)
    check_close(first, ref, K, wl.F16)
    absum = oracle.gemm_absum_matmul(A, B, M, N, K, wl.F16, transB)
    assert np.all(np.abs(first - ref) <= fp32_sum_bound(absum, ref, K, unit_roundoff(wl.F16)))
    for fill in (0.0, -1.0e30):
        assert np.array_equal(run_ws(A, B, M, N, K, wl.F16, wl.F16, transB, ws_fill=fill), first)
    Ad, Bd = to_device(A, wl.F16, (M, K)), to_device(B, wl.F16, wl.b_shape(M, N, K, transB))
    need = gr.gemm_relu_workspace_size(M, N, K, wl.F16, wl.F16, transB)
    ws = _ws(need)
    outs = [out_tensor(M, N, wl.F16, float("nan")) for _ in range(4)]
    for C in outs:
        gr.gemm_relu_ws(Ad, Bd, C, M, N, K, wl.F16, wl.F16, transB, ws, need)
    torch.cuda.synchronize()
    assert counters_zero(ws)
    for C in outs:
        assert np.array_equal(from_device(C), first)


@pytest.mark.gpu
@need_sk
@pytest.mark.parametrize("name", ["gemm_relu_bf16_tB_f32_4096x7168x4096", "gemm_relu_f16_4097x3001x5003"])
def test_workload_full_size_every_output(name, monkeypatch):
    """The workloads whose last round of 256x256 tiles is partial, split this
    way: every output against the oracle, on integer inputs bit for bit and
    on the uniform inputs within the bounds."""
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", SK)
    w = wl.WORKLOADS[name]
    M, N, K, ic, oc, tb = w["M"], w["N"], w["K"], w["in_dtype"], w["out_dtype"], w["transB"]
    Ai, Bi = wl.workload_inputs(name, int_values=True)
    goti = run_ws(Ai, Bi, M, N, K, ic, oc, tb, ws_fill=float("nan"))
    assert np.array_equal(goti, oracle.gemm_relu_ref_matmul(Ai, Bi, M, N, K, ic, tb))
    A, B = wl.workload_inputs(name)
    got = run_ws(A, B, M, N, K, ic, oc, tb)
    ref = oracle.gemm_relu_ref_matmul(A, B, M, N, K, ic, tb)
    check_close(got, ref, K, oc)
    absum = oracle.gemm_absum_matmul(A, B, M, N, K, ic, tb)
    assert np.all(np.abs(got - ref) <= fp32_sum_bound(absum, ref, K, unit_roundoff(oc)))


@pytest.mark.gpu
@need_sk
def test_alternating_inputs_on_one_workspace(monkeypatch):
    """Back-to-back calls on one workspace whose inputs alternate between two
    sets: every result must be its own inputs' product (a piece that read
    another call's partial would show here)."""
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", SK)
    import torch
    M, N, K = 2560, 5120, 2048        # 10 x 20 = 200 tiles, all split over 256 units
    sets = []
    for k in range(2):
        A, B = int_inputs(M, N, K, wl.F16, 1, 820 + 10 * k, wl.F16)
        sets.append((to_device(A, wl.F16, (M, K)), to_device(B, wl.F16, (N, K)),
                     oracle.gemm_relu_ref_matmul(A, B, M, N, K, wl.F16, 1)))
    assert not np.array_equal(sets[0][2], sets[1][2])
    need = gr.gemm_relu_workspace_size(M, N, K, wl.F16, wl.F16, 1)
    assert need == need_bytes(256)
    ws = _ws(need, float("nan"))
    Cd0 = out_tensor(M, N, wl.F16, float("nan"))
    assert gr.gemm_relu_ws_plan(sets[0][0], sets[0][1], Cd0, M, N, K, wl.F16, wl.F16, 1, ws, need) == SK
    outs = []
    for call in range(12):
        Ad, Bd, _ = sets[call % 2]
        Cd = out_tensor(M, N, wl.F16, float("nan"))
        gr.gemm_relu_ws(Ad, Bd, Cd, M, N, K, wl.F16, wl.F16, 1, ws, need)
        outs.append(Cd)
    torch.cuda.synchronize()
    assert counters_zero(ws)
    for call, Cd in enumerate(outs):
        assert np.array_equal(from_device(Cd), sets[call % 2][2]), call
