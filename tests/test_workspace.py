"""gemm_relu_ws: the K split with a caller's workspace.

The product is gemm_relu's (page "TileLang：GPU/NPU 通用算子 DSL", §3.2); the
split only changes the order in which the fp32 accumulator is formed (per part,
then the parts in K order) and applies the ReLU once, to the whole sum.  So the
bars are gemm_relu's: bit for bit on integer inputs, the contract bound and the
fp32-summation bound on random ones, against the oracle.

Host-side tests (plan choice, workspace size, argument checks) run on the CPU;
the rest need the GPU.
"""
import numpy as np
import pytest

import dense_tiled_gemm_relu_amd as gr
import oracle
import workloads as wl
from tests.helpers import (check_close, from_device, fp32_sum_bound, out_tensor, to_device,
                           unit_roundoff)

SPLITK = "d64x128x64_s4_splitk"
SKINNY = "d32x64x128_s4"
FAKE = 1 << 40          # host-side plans: aligned, disjoint fake addresses


def fake_args(M, N, K, in_code=wl.F16, out_code=wl.F16):
    eb = 1 if in_code in (wl.F8E4M3, wl.F8E5M2) else 2
    a = FAKE
    b = a + M * K * eb + 4096
    c = b + K * N * eb + 4096
    w = ((c + M * N * 4 + 4096) + 255) // 256 * 256
    return a, b, c, w


FLAG_BYTES = 4096      # the workspace's arrival counters, before the partial tiles


def need_bytes(M, N, parts):
    """Counters, then one fp32 64 x 128 partial tile per tile and part."""
    return FLAG_BYTES + parts * (-(-M // 64)) * (-(-N // 128)) * 64 * 128 * 4


# ------------------------------------------------------------ host side
def test_workspace_size_of_the_skinny_workload():
    # 64 x 8192: 64 tiles of 64 x 128, so 4 parts of 2048 k (32 steps of 64)
    assert gr.gemm_relu_workspace_size(64, 8192, 8192, wl.F16, wl.F16, 0) == need_bytes(64, 8192, 4)
    assert need_bytes(64, 8192, 4) == 4096 + 8 * 2 ** 20
    assert gr.gemm_relu_workspace_size(64, 8192, 8192, wl.BF16, wl.F32, 0) == need_bytes(64, 8192, 4)
    # B stored (N,K): the 32 x 64 tiles fill the CUs at N = 8192, not at N = 4096
    assert gr.gemm_relu_workspace_size(64, 8192, 8192, wl.BF16, wl.F32, 1) == 0
    assert gr.gemm_relu_workspace_size(64, 4096, 8192, wl.BF16, wl.F32, 1) == need_bytes(64, 4096, 8)
    # fewer rows take the same 64-row tiles
    assert gr.gemm_relu_workspace_size(16, 8192, 8192, wl.F16, wl.F16, 0) == need_bytes(16, 8192, 4)
    # 64 x 4096 x 16384: 32 tiles, 8 parts
    assert gr.gemm_relu_workspace_size(64, 4096, 16384, wl.F16, wl.F16, 0) == need_bytes(64, 4096, 8)
    # 8-bit inputs: 128-element steps, the same part count
    assert gr.gemm_relu_workspace_size(64, 8192, 8192, wl.F8E4M3, wl.F16, 0) == need_bytes(64, 8192, 4)


@pytest.mark.parametrize("M,N,K", [(8192, 8192, 8192), (128, 8192, 8192), (64, 8192, 256),
                                   (64, 100, 8192), (0, 64, 64), (64, 0, 64), (64, 8192, 0),
                                   (4096, 7168, 4096), (4096, 4096, 4096)])
def test_no_split_where_it_does_not_pay(M, N, K):
    """Large M, many tiles, short K, N below one (K,N) tile, empty: no split."""
    assert gr.gemm_relu_workspace_size(M, N, K, wl.F16, wl.F16, 0) == 0


def test_workspace_size_rejects_bad_codes():
    assert gr.gemm_relu_workspace_size(-1, 8, 8, wl.F16, wl.F16, 0) == gr.EINVAL
    assert gr.gemm_relu_workspace_size(8, 8, 8, 99, wl.F16, 0) == gr.EINVAL
    assert gr.gemm_relu_workspace_size(8, 8, 8, wl.F16, wl.F8E4M3, 0) == gr.EINVAL
    assert gr.gemm_relu_workspace_size(8, 8, 8, wl.F16, wl.F16, 2) == gr.EINVAL


def test_ws_plan_choice():
    M, N, K = 64, 8192, 8192
    a, b, c, w = fake_args(M, N, K)
    need = gr.gemm_relu_workspace_size(M, N, K, wl.F16, wl.F16, 0)
    assert gr.gemm_relu_ws_plan(a, b, c, M, N, K, wl.F16, wl.F16, 0, w, need) == SPLITK
    assert gr.gemm_relu_ws_plan(a, b, c, M, N, K, wl.F16, wl.F16, 1, w, need) == SKINNY
    assert gr.gemm_relu_ws_plan(a, b, c, M, 4096, K, wl.F16, wl.F16, 1, w, need) == SPLITK
    # too small a workspace, or none: the workspace-free plan
    assert gr.gemm_relu_ws_plan(a, b, c, M, N, K, wl.F16, wl.F16, 0, w, need - 1) == SKINNY
    assert gr.gemm_relu_ws_plan(a, b, c, M, N, K, wl.F16, wl.F16, 0, None, need) == SKINNY
    assert gr.gemm_relu_ws_plan(a, b, c, M, N, K, wl.F16, wl.F16, 0, w, 0) == SKINNY
    assert gr.gemm_relu_plan(a, b, c, M, N, K, wl.F16, wl.F16, 0) == SKINNY
    # the square headline shape never splits
    a, b, c, w = fake_args(8192, 8192, 8192)
    assert gr.gemm_relu_ws_plan(a, b, c, 8192, 8192, 8192, wl.F16, wl.F16, 0, w,
                                1 << 30) == "d256x256x32_s4_i16w8"


def test_ws_plan_rejects_bad_workspaces():
    M, N, K = 64, 8192, 8192
    a, b, c, w = fake_args(M, N, K)
    need = gr.gemm_relu_workspace_size(M, N, K, wl.F16, wl.F16, 0)
    assert gr.gemm_relu_ws_plan(a, b, c, M, N, K, wl.F16, wl.F16, 0, w + 16, need) is None
    assert gr.gemm_relu_ws_plan(a, b, c, M, N, K, wl.F16, wl.F16, 0, c, need) is None     # over C
    assert gr.gemm_relu_ws_plan(a, b, c, M, N, K, wl.F16, wl.F16, 0, a, need) is None     # over A
    assert gr.gemm_relu_ws_plan(a, b, c, M, N, K, wl.F16, wl.F16, 0, b - 256, need) is None
    # the call itself checks the same before touching the device
    assert gr.gemm_relu_ws_status(a, b, c, M, N, K, wl.F16, wl.F16, 0, w + 16, need, 0) == gr.EINVAL
    assert gr.gemm_relu_ws_status(a, b, c, M, N, K, wl.F16, wl.F16, 0, c, need, 0) == gr.EINVAL


def test_forced_split_and_part_count(monkeypatch):
    M, N, K = 200, 300, 1000
    a, b, c, w = fake_args(M, N, K)
    assert gr.gemm_relu_ws_plan(a, b, c, M, N, K, wl.F16, wl.F16, 0, w, 1 << 30) != SPLITK
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", SPLITK)
    assert gr.gemm_relu_ws_plan(a, b, c, M, N, K, wl.F16, wl.F16, 0, w, 1 << 30) == SPLITK
    # 12 tiles: 16 parts of one 64-element step each (16 steps)
    assert gr.gemm_relu_workspace_size(M, N, K, wl.F16, wl.F16, 0) == need_bytes(M, N, 16)
    monkeypatch.setenv("GEMM_RELU_SPLITK_PARTS", "3")
    assert gr.gemm_relu_workspace_size(M, N, K, wl.F16, wl.F16, 0) == need_bytes(M, N, 3)
    # 16 steps in parts of ceil(16 / 7) = 3: 6 parts, all non-empty
    monkeypatch.setenv("GEMM_RELU_SPLITK_PARTS", "7")
    assert gr.gemm_relu_workspace_size(M, N, K, wl.F16, wl.F16, 0) == need_bytes(M, N, 6)
    # one step: nothing to split
    assert gr.gemm_relu_workspace_size(M, N, 64, wl.F16, wl.F16, 0) == 0
    # more than 1024 tiles: no split even when forced
    assert gr.gemm_relu_workspace_size(4096, 4096, 4096, wl.F16, wl.F16, 0) == 0


# ------------------------------------------------------------ GPU
def _ws(nbytes, fill=None):
    """A zeroed workspace (its counters must start at zero); the partial-tile
    region optionally filled with garbage, which the call must not read."""
    import torch
    t = torch.zeros(max(nbytes, FLAG_BYTES), dtype=torch.uint8, device="cuda")
    assert t.data_ptr() % 256 == 0
    if fill is not None and t.numel() > FLAG_BYTES:
        t[FLAG_BYTES:].view(torch.float32).fill_(fill)
    return t


def counters_zero(ws):
    return bool((ws[:FLAG_BYTES] == 0).all())


def run_ws(A, B, M, N, K, in_code, out_code, transB, expect_plan=SPLITK, ws_fill=None):
    import torch
    Ad, Bd = to_device(A, in_code, (M, K)), to_device(B, in_code, wl.b_shape(M, N, K, transB))
    Cd = out_tensor(M, N, out_code, float("nan"))
    need = gr.gemm_relu_workspace_size(M, N, K, in_code, out_code, transB)
    ws = _ws(need, ws_fill)
    assert gr.gemm_relu_ws_plan(Ad, Bd, Cd, M, N, K, in_code, out_code, transB, ws,
                                ws.numel()) == expect_plan
    gr.gemm_relu_ws(Ad, Bd, Cd, M, N, K, in_code, out_code, transB, ws, ws.numel())
    torch.cuda.synchronize()
    assert counters_zero(ws)
    return from_device(Cd)


def int_inputs(M, N, K, in_code, transB, seed, out_code):
    lo, hi = (-1, 1) if out_code == wl.BF16 else (-2, 2)
    return (wl.integers((M, K), seed, in_code, lo, hi),
            wl.integers(wl.b_shape(M, N, K, transB), seed + 1, in_code, lo, hi))


EXACT = {wl.F16: 2048.0, wl.BF16: 256.0, wl.F32: 2.0 ** 24}
COMBOS = [(i, o) for i in (wl.F16, wl.BF16) for o in (wl.F16, wl.BF16, wl.F32)] + \
         [(wl.F8E4M3, wl.F16), (wl.F8E5M2, wl.F32)]
# forced split: several tiles both ways, M and N tails, K tails (K % 64 != 0),
# one tile row of one row, N below two tiles
FORCED_SHAPES = [(200, 300, 1000), (64, 520, 4103), (1, 128, 777), (130, 129, 2049),
                 (37, 1000, 3000)]


@pytest.mark.gpu
@pytest.mark.parametrize("in_code,out_code", COMBOS)
@pytest.mark.parametrize("transB", [0, 1])
@pytest.mark.parametrize("shape", FORCED_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_forced_split_integer_bitexact(in_code, out_code, transB, shape, monkeypatch):
    M, N, K = shape
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", SPLITK)
    A, B = int_inputs(M, N, K, in_code, transB, 700, out_code)
    ref = oracle.gemm_relu_ref_matmul(A, B, M, N, K, in_code, transB)
    assert np.abs(ref).max() < EXACT[out_code]
    got = run_ws(A, B, M, N, K, in_code, out_code, transB, ws_fill=float("nan"))
    assert np.array_equal(got, ref)
    assert not np.any(np.signbit(got))


@pytest.mark.gpu
@pytest.mark.parametrize("parts", [2, 3, 5, 16])
@pytest.mark.parametrize("transB", [0, 1])
def test_part_counts_integer_bitexact(parts, transB, monkeypatch):
    """Parts of unequal length (the last one shorter, and with the K tail)."""
    M, N, K = 64, 1024, 64 * 21 + 13
    monkeypatch.setenv("GEMM_RELU_SPLITK_PARTS", str(parts))
    A, B = int_inputs(M, N, K, wl.F16, transB, 710, wl.F16)
    ref = oracle.gemm_relu_ref_matmul(A, B, M, N, K, wl.F16, transB)
    got = run_ws(A, B, M, N, K, wl.F16, wl.F16, transB, ws_fill=float("inf"))
    assert np.array_equal(got, ref)


@pytest.mark.gpu
@pytest.mark.parametrize("in_code,out_code", COMBOS)
@pytest.mark.parametrize("transB", [0, 1])
def test_uniform_within_bounds(in_code, out_code, transB, monkeypatch):
    M, N, K = 48, 2048, 6000
    A = wl.uniform((M, K), 720, in_code)
    B = wl.uniform(wl.b_shape(M, N, K, transB), 721, in_code)
    got = run_ws(A, B, M, N, K, in_code, out_code, transB)
    ref = oracle.gemm_relu_ref(A, B, M, N, K, in_code, transB)
    check_close(got, ref, K, out_code)
    absum = oracle.gemm_absum_matmul(A, B, M, N, K, in_code, transB)
    assert np.all(np.abs(got - ref) <= fp32_sum_bound(absum, ref, K, unit_roundoff(out_code)))


@pytest.mark.gpu
def test_skinny_workload_full_size_every_output():
    """64 x 8192 x 8192 fp16 (the skinny workload), as the workload table times
    it with a workspace: every output against the oracle."""
    name = "gemm_relu_f16_64x8192x8192"
    w = wl.WORKLOADS[name]
    M, N, K, ic, oc, tb = w["M"], w["N"], w["K"], w["in_dtype"], w["out_dtype"], w["transB"]
    A, B = wl.workload_inputs(name)
    got = run_ws(A, B, M, N, K, ic, oc, tb)
    ref = oracle.gemm_relu_ref(A, B, M, N, K, ic, tb)
    check_close(got, ref, K, oc)
    absum = oracle.gemm_absum_matmul(A, B, M, N, K, ic, tb)
    assert np.all(np.abs(got - ref) <= fp32_sum_bound(absum, ref, K, unit_roundoff(oc)))
    Ai, Bi = wl.workload_inputs(name, int_values=True)
    goti = run_ws(Ai, Bi, M, N, K, ic, oc, tb)
    assert np.array_equal(goti, oracle.gemm_relu_ref_matmul(Ai, Bi, M, N, K, ic, tb))


@pytest.mark.gpu
def test_repeatable_and_workspace_contents_ignored():
    """Same bits on every call, whatever the workspace held before."""
    import torch
    M, N, K = 64, 4096, 8192
    A = wl.uniform((M, K), 730, wl.F16)
    B = wl.uniform((K, N), 731, wl.F16)
    first = run_ws(A, B, M, N, K, wl.F16, wl.F16, 0, ws_fill=float("nan"))
    for fill in (0.0, -1.0e30, float("-inf")):
        again = run_ws(A, B, M, N, K, wl.F16, wl.F16, 0, ws_fill=fill)
        assert np.array_equal(first, again)
    # and one workspace reused by back-to-back calls on one stream
    Ad, Bd = to_device(A, wl.F16, (M, K)), to_device(B, wl.F16, (K, N))
    ws = _ws(gr.gemm_relu_workspace_size(M, N, K, wl.F16, wl.F16, 0))
    outs = [out_tensor(M, N, wl.F16, float("nan")) for _ in range(3)]
    for C in outs:
        gr.gemm_relu_ws(Ad, Bd, C, M, N, K, wl.F16, wl.F16, 0, ws, ws.numel())
    torch.cuda.synchronize()
    for C in outs:
        assert np.array_equal(from_device(C), first)
    assert counters_zero(ws)


@pytest.mark.gpu
def test_one_workspace_for_shapes_and_part_counts_in_turn(monkeypatch):
    """Calls of different tile and part counts share one workspace, back to
    back on one stream: each leaves the counters as the next needs them."""
    import torch
    shapes = [(64, 8192, 4096, 0), (40, 1000, 3000, 1), (64, 4096, 16384, 0), (1, 256, 2048, 0),
              (64, 4096, 8192, 1)]
    big = max(gr.gemm_relu_workspace_size(M, N, K, wl.F16, wl.F16, tb) for M, N, K, tb in shapes)
    ws = _ws(big, float("nan"))
    pending = []
    for idx, (M, N, K, tb) in enumerate(shapes):
        A, B = int_inputs(M, N, K, wl.F16, tb, 750 + 2 * idx, wl.F16)
        Ad, Bd = to_device(A, wl.F16, (M, K)), to_device(B, wl.F16, wl.b_shape(M, N, K, tb))
        Cd = out_tensor(M, N, wl.F16, float("nan"))
        assert gr.gemm_relu_ws_plan(Ad, Bd, Cd, M, N, K, wl.F16, wl.F16, tb, ws, big) == SPLITK
        gr.gemm_relu_ws(Ad, Bd, Cd, M, N, K, wl.F16, wl.F16, tb, ws, big)
        pending.append((A, B, M, N, K, tb, Cd, Ad, Bd))
    torch.cuda.synchronize()
    assert counters_zero(ws)
    for A, B, M, N, K, tb, Cd, _, _ in pending:
        assert np.array_equal(from_device(Cd), oracle.gemm_relu_ref_matmul(A, B, M, N, K, wl.F16, tb))


@pytest.mark.gpu
def test_small_workspace_runs_the_workspace_free_plan():
    import torch
    M, N, K = 64, 8192, 4096
    A, B = int_inputs(M, N, K, wl.F16, 0, 740, wl.F16)
    Ad, Bd = to_device(A, wl.F16, (M, K)), to_device(B, wl.F16, (K, N))
    Cd = out_tensor(M, N, wl.F16, float("nan"))
    ws = _ws(4096)
    assert gr.gemm_relu_ws_plan(Ad, Bd, Cd, M, N, K, wl.F16, wl.F16, 0, ws, 4096) == SKINNY
    gr.gemm_relu_ws(Ad, Bd, Cd, M, N, K, wl.F16, wl.F16, 0, ws, 4096)
    torch.cuda.synchronize()
    assert np.array_equal(from_device(Cd), oracle.gemm_relu_ref_matmul(A, B, M, N, K, wl.F16, 0))


@pytest.mark.gpu
@pytest.mark.parametrize("transB", [0, 1])
def test_alternating_inputs_on_one_workspace(transB):
    """Back-to-back calls on one workspace whose inputs alternate between two
    sets: every result must be its own inputs' product (a part that read
    another call's partial tile would show here), for parts on any XCD."""
    import torch
    M, N, K = 64, 4096, 4096
    sets = []
    for k in range(2):
        A, B = int_inputs(M, N, K, wl.F16, transB, 760 + 10 * k, wl.F16)
        sets.append((A, B, to_device(A, wl.F16, (M, K)), to_device(B, wl.F16, wl.b_shape(M, N, K, transB)),
                     oracle.gemm_relu_ref_matmul(A, B, M, N, K, wl.F16, transB)))
    assert not np.array_equal(sets[0][4], sets[1][4])
    need = gr.gemm_relu_workspace_size(M, N, K, wl.F16, wl.F16, transB)
    ws = _ws(need, float("nan"))
    outs = []
    for call in range(24):
        _, _, Ad, Bd, _ = sets[call % 2]
        Cd = out_tensor(M, N, wl.F16, float("nan"))
        gr.gemm_relu_ws(Ad, Bd, Cd, M, N, K, wl.F16, wl.F16, transB, ws, need)
        outs.append(Cd)
    torch.cuda.synchronize()
    assert counters_zero(ws)
    for call, Cd in enumerate(outs):
        assert np.array_equal(from_device(Cd), sets[call % 2][4]), call
