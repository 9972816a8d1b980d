"""Block-scaled (OCP MX) GEMM + ReLU through the C-ABI (gemm_relu_mx) against
the oracle: the MXFP8 / MXFP4 items of page "TileLang：GPU/NPU 通用算子 DSL",
§4.1, read as the OCP Microscaling definition (one E8M0 scale per 32 elements
along K for A (M,K) and for B stored (N,K))."""
import numpy as np
import pytest

import dense_tiled_gemm_relu_amd as gr
import oracle
import workloads as wl
from tests.helpers import (built_configs, check_close, from_device, fp32_sum_bound, out_tensor,
                           unit_roundoff)

pytestmark = pytest.mark.gpu

FMTS = [wl.MX_E4M3, wl.MX_E5M2, wl.MX_E2M1]
# the interleaved four-stage tile stages scales in LDS by 16 blocks of a row,
# so it serves K >= 512 only
INTERLEAVED = "d256x256x32_s4_i"
CONFIGS = built_configs([INTERLEAVED, "d256x256x64_s2", "d256x128x64_s2", "d128x128x64_s2"])


def _needs(cfg, K):
    if cfg == INTERLEAVED and K < 512:
        pytest.skip("the interleaved tile needs K >= 512 (16 scale blocks per row)")


@pytest.fixture(autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    yield


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).reshape(-1)).cuda()


def run_mx(A, SA, B, SB, M, N, K, fmt, out_code, cfg=None, monkeypatch=None):
    import torch
    if cfg is not None:
        monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", cfg)
    Ad, SAd, Bd, SBd = _dev(A), _dev(SA), _dev(B), _dev(SB)
    Cd = out_tensor(M, N, out_code)
    if cfg is not None:
        assert gr.gemm_relu_mx_plan(Ad, SAd, Bd, SBd, Cd, M, N, K, fmt, out_code) == cfg
    gr.gemm_relu_mx(Ad, SAd, Bd, SBd, Cd, M, N, K, fmt, out_code)
    torch.cuda.synchronize()
    return from_device(Cd)


def int_mx(M, N, K, fmt, seed, scale_choices=(127,), top=2):
    """Integer elements in {-top..top} (exact in every format) and scales
    drawn from scale_choices."""
    rng = np.random.default_rng(seed)
    a = rng.integers(-top, top + 1, size=(M, K)).astype(np.float64)
    b = rng.integers(-top, top + 1, size=(N, K)).astype(np.float64)
    if fmt == wl.MX_E2M1:
        A, B = wl.pack_e2m1(wl.e2m1_codes(a)), wl.pack_e2m1(wl.e2m1_codes(b))
    else:
        plain = wl.F8E4M3 if fmt == wl.MX_E4M3 else wl.F8E5M2
        A, B = wl.encode(a, plain), wl.encode(b, plain)
    SA = rng.choice(scale_choices, size=(M, K // 32)).astype(np.uint8)
    SB = rng.choice(scale_choices, size=(N, K // 32)).astype(np.uint8)
    return A, SA, B, SB


@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("out_code", [wl.F16, wl.BF16, wl.F32])
@pytest.mark.parametrize("shape", [(264, 520, 288), (301, 517, 224), (264, 520, 1120)],
                         ids=["tail32", "ragged", "long"])
def test_mx_integer_unit_scales_bitexact(cfg, fmt, out_code, shape, monkeypatch):
    M, N, K = shape
    _needs(cfg, K)
    # a bf16 C holds every integer only up to 256: elements in {-1, 0, 1} keep
    # |C| below it (about 4.5 standard deviations of sqrt(4K/9) at K = 1120)
    A, SA, B, SB = int_mx(M, N, K, fmt, 900 + fmt, top=1 if out_code == wl.BF16 else 2)
    ref = oracle.gemm_relu_mx_ref(A, SA, B, SB, M, N, K, fmt)
    assert np.abs(ref).max() < (256 if out_code == wl.BF16 else 2048)
    got = run_mx(A, SA, B, SB, M, N, K, fmt, out_code, cfg, monkeypatch)
    assert np.array_equal(got, ref)
    assert not np.any(np.signbit(got))


@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("fmt", FMTS)
def test_mx_scaled_blocks_bitexact(cfg, fmt, monkeypatch):
    """Per-block scales 2^-1, 2^0, 2^1 on integer elements: every sum is exact
    in fp32, so an fp32 C must equal the oracle bit for bit — any block, row or
    lane-group mix-up of the scales shows.  K spans 17 steps of 64 storage
    bytes plus a tail, so the four-stage ring runs its steady loop."""
    M, N, K = 200, 330, 1120
    A, SA, B, SB = int_mx(M, N, K, fmt, 910 + fmt, scale_choices=(126, 127, 128))
    ref = oracle.gemm_relu_mx_ref(A, SA, B, SB, M, N, K, fmt)
    got = run_mx(A, SA, B, SB, M, N, K, fmt, wl.F32, cfg, monkeypatch)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("K", [512, 544, 2016, 4128])
@pytest.mark.parametrize("fmt", FMTS)
def test_mx_interleaved_scale_groups(K, fmt, monkeypatch):
    """The interleaved tile's LDS scale groups (16 blocks of a row per group):
    one group exactly, a tail past it, and rows whose last group is partial
    and moved back (K / 32 = 63, 129), with per-block scales on integer
    elements (exact in fp32)."""
    M, N = 300, 280
    A, SA, B, SB = int_mx(M, N, K, fmt, 960 + K + fmt, scale_choices=(126, 127, 128))
    ref = oracle.gemm_relu_mx_ref(A, SA, B, SB, M, N, K, fmt)
    got = run_mx(A, SA, B, SB, M, N, K, fmt, wl.F32, INTERLEAVED, monkeypatch)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("fmt", FMTS)
def test_mx_coded_scales(fmt):
    """All elements 1 and one distinct power-of-two scale per (row, block): each
    output is sum_b 32 2^(ea[i][b] + eb[j][b]), so it names its blocks."""
    M, N, K = 96, 160, 256
    rng = np.random.default_rng(920 + fmt)
    ones_a = np.ones((M, K))
    ones_b = np.ones((N, K))
    if fmt == wl.MX_E2M1:
        A, B = wl.pack_e2m1(wl.e2m1_codes(ones_a)), wl.pack_e2m1(wl.e2m1_codes(ones_b))
    else:
        plain = wl.F8E4M3 if fmt == wl.MX_E4M3 else wl.F8E5M2
        A, B = wl.encode(ones_a, plain), wl.encode(ones_b, plain)
    # exponents within +-3: every sum of 8 blocks stays exact in fp32
    SA = (127 + rng.integers(-3, 4, size=(M, K // 32))).astype(np.uint8)
    SB = (127 + rng.integers(-3, 4, size=(N, K // 32))).astype(np.uint8)
    ref = oracle.gemm_relu_mx_ref(A, SA, B, SB, M, N, K, fmt)
    got = run_mx(A, SA, B, SB, M, N, K, fmt, wl.F32)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("fmt", FMTS)
def test_mx_quantized_uniform_tolerance(cfg, fmt, monkeypatch):
    M, N, K = 331, 263, 640
    _needs(cfg, K)
    A, SA, B, SB = wl.mx_inputs(M, N, K, fmt, 930)
    got = run_mx(A, SA, B, SB, M, N, K, fmt, wl.F16, cfg, monkeypatch)
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ref, absum = oracle.gemm_relu_mx_ref(A, SA, B, SB, M, N, K, fmt,
                                         rows=rows.ravel(), cols=cols.ravel())
    ref, absum = ref.reshape(M, N), absum.reshape(M, N)
    check_close(got, ref, K, wl.F16)
    assert np.all(np.abs(got - ref) <= fp32_sum_bound(absum, ref, K, unit_roundoff(wl.F16)))


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (5, 300, 32), (257, 3, 96), (64, 64, 0),
                                   (130, 129, 4096 + 32)])
@pytest.mark.parametrize("fmt", FMTS)
def test_mx_edge_shapes(M, N, K, fmt):
    A, SA, B, SB = int_mx(M, N, K, fmt, 940 + M + N)
    ref = oracle.gemm_relu_mx_ref(A, SA, B, SB, M, N, K, fmt)
    got = run_mx(A, SA, B, SB, M, N, K, fmt, wl.F32)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("fmt", FMTS)
def test_mx_workload_full_size(fmt):
    """8192^3 on sampled outputs against the oracle's dot products."""
    M = N = K = 8192
    A, SA, B, SB = wl.mx_inputs(M, N, K, fmt, 950)
    got = run_mx(A, SA, B, SB, M, N, K, fmt, wl.F16)
    rng = np.random.default_rng(951)
    rows = np.concatenate([rng.integers(0, M, 1024), np.zeros(32, int), np.full(32, M - 1)])
    cols = np.concatenate([rng.integers(0, N, 1024), rng.integers(0, N, 64)])
    ref, absum = oracle.gemm_relu_mx_ref(A, SA, B, SB, M, N, K, fmt, rows=rows, cols=cols)
    check_close(got[rows, cols], ref, K, wl.F16)
    assert np.all(np.abs(got[rows, cols] - ref) <=
                  fp32_sum_bound(absum, ref, K, unit_roundoff(wl.F16)))
    frac0 = float(np.mean(got == 0.0))
    assert 0.4 < frac0 < 0.6
