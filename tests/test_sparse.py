"""2:4 structured-sparse GEMM + ReLU through the C-ABI (gemm_relu_sp) against
the oracle: the T.gemm_sp item of page "TileLang：GPU/NPU 通用算子 DSL", §4.1,
with A compressed and its metadata loaded beside it (page "从 TVM 到
TileLang…", §四).  Format: As (M, K/2) stored values, E nibbles p0 | p1 << 2
blocked by 64 columns of K (M x 8 bytes per block)."""
import numpy as np
import pytest

import dense_tiled_gemm_relu_amd as gr
import oracle
import workloads as wl
from tests.helpers import (built_configs, check_close, from_device, fp32_sum_bound, out_tensor,
                           unit_roundoff)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    yield


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).reshape(-1)).cuda()


SP = "sp256x256x64_s3_w8"
# the plan's configuration (2 x 4 waves), and in a comparison build its 2 x 2-wave variant
SP_CONFIGS = built_configs([SP, "sp256x256x64_s3"])


def run_sp(As, E, B, M, N, K, in_dtype, out_code, transB, cfg=SP, monkeypatch=None):
    import torch
    if cfg != SP:
        monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", cfg)
    Ad, Ed, Bd = _dev(As), _dev(E), _dev(B)
    Cd = out_tensor(M, N, out_code)
    assert gr.gemm_relu_sp_plan(Ad, Ed, Bd, Cd, M, N, K, in_dtype, out_code, transB) == cfg
    gr.gemm_relu_sp(Ad, Ed, Bd, Cd, M, N, K, in_dtype, out_code, transB)
    torch.cuda.synchronize()
    return from_device(Cd)


@pytest.mark.parametrize("cfg", SP_CONFIGS)
@pytest.mark.parametrize("in_dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("out_code", [wl.F16, wl.BF16, wl.F32])
@pytest.mark.parametrize("transB", [0, 1])
@pytest.mark.parametrize("shape", [(256, 256, 64), (264, 520, 288), (301, 517, 200),
                                   (300, 300, 1100)],
                         ids=["one_tile", "tail32", "ragged", "long"])
def test_sp_integer_bitexact(cfg, in_dtype, out_code, transB, shape, monkeypatch):
    M, N, K = shape
    if out_code == wl.BF16:
        K = 64 + 4 * (K % 3)                    # keep |C| inside bf16's exact integers
    As, E, B = wl.sp_inputs(M, N, K, in_dtype, transB, 70, int_values=True)
    ref = oracle.gemm_relu_sp_ref(As, E, B, M, N, K, in_dtype, transB)
    got = run_sp(As, E, B, M, N, K, in_dtype, out_code, transB, cfg, monkeypatch)
    assert np.array_equal(got, ref)
    assert not np.any(np.signbit(got))


@pytest.mark.parametrize("in_dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("transB", [0, 1])
def test_sp_uniform_tolerance(in_dtype, transB):
    M, N, K = 331, 263 if transB else 300, 1028
    As, E, B = wl.sp_inputs(M, N, K, in_dtype, transB, 71)
    got = run_sp(As, E, B, M, N, K, in_dtype, wl.F32, transB)
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ref, absum = oracle.gemm_relu_sp_ref(As, E, B, M, N, K, in_dtype, transB,
                                         rows=rows.ravel(), cols=cols.ravel())
    ref, absum = ref.reshape(M, N), absum.reshape(M, N)
    assert np.all(np.abs(got - ref) <= fp32_sum_bound(absum, ref, K, unit_roundoff(wl.F32)))


def test_sp_every_position_pair():
    """Each row of A keeps one fixed position pair in every group (all six
    pairs over six rows) and B's row k holds k: C[i][j] names the positions."""
    M, N, K = 6, 256, 64
    positions = np.zeros((M, K // 4, 2), np.int64)
    for i, (p0, p1) in enumerate(wl.SP_PAIRS):
        positions[i, :, 0], positions[i, :, 1] = p0, p1
    vals = np.tile([1.0, 2.0], (M, K // 4))
    As, E = wl.encode(vals, wl.F16), wl.sp_pack(positions, M, K)
    b = np.tile(np.arange(K, dtype=np.float64)[:, None], (1, N))
    B = wl.encode(b, wl.F16)
    got = run_sp(As, E, B, M, N, K, wl.F16, wl.F32, 0)
    q = np.arange(K // 4)
    want = np.array([(4 * q + p0 + 2 * (4 * q + p1)).sum() for p0, p1 in wl.SP_PAIRS], dtype=float)
    assert np.array_equal(got, np.repeat(want[:, None], N, axis=1))


@pytest.mark.parametrize("M,N,K,transB", [(1, 1, 4, 1), (5, 300, 8, 0), (257, 3, 12, 1),
                                          (64, 256, 0, 0), (130, 257, 4096 + 4, 1)])
def test_sp_edge_shapes(M, N, K, transB):
    As, E, B = wl.sp_inputs(M, N, K, wl.F16, transB, 72, int_values=True)
    ref = oracle.gemm_relu_sp_ref(As, E, B, M, N, K, wl.F16, transB)
    got = run_sp(As, E, B, M, N, K, wl.F16, wl.F32, transB)
    assert np.array_equal(got, ref)


def test_sp_empty_is_a_no_op():
    import torch
    C = torch.full((4, 4), 7.0, dtype=torch.float32, device="cuda")
    gr.gemm_relu_sp(0, 0, 0, C, 0, 4, 8, wl.F16, wl.F32, 0)
    torch.cuda.synchronize()
    assert torch.all(C == 7.0)


def test_sp_workload_full_size():
    """8192^3 on sampled outputs against the oracle's dot products."""
    w = wl.WORKLOADS["gemm_relu_sp_f16_8192"]
    M, N, K, tb = w["M"], w["N"], w["K"], w["transB"]
    As, E, B = wl.sp_inputs(M, N, K, w["in_dtype"], tb, w["index"])
    got = run_sp(As, E, B, M, N, K, w["in_dtype"], w["out_dtype"], tb)
    rng = np.random.default_rng(73)
    rows = np.concatenate([rng.integers(0, M, 1024), np.zeros(32, int), np.full(32, M - 1)])
    cols = np.concatenate([rng.integers(0, N, 1024), rng.integers(0, N, 64)])
    ref, absum = oracle.gemm_relu_sp_ref(As, E, B, M, N, K, w["in_dtype"], tb, rows=rows, cols=cols)
    check_close(got[rows, cols], ref, K, w["out_dtype"])
    assert np.all(np.abs(got[rows, cols] - ref) <=
                  fp32_sum_bound(absum, ref, K, unit_roundoff(w["out_dtype"])))
    frac0 = float(np.mean(got == 0.0))
    assert 0.4 < frac0 < 0.6
