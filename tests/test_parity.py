"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

Integer-valued inputs have exactly one correct result (every partial sum is an
integer far below 2^24, so fp32 accumulation is exact in any order): those
cases are compared bit for bit.  Random inputs are compared element by element
with the bound |gpu - ref| <= 2^-9 |ref| + 1e-3 sqrt(K) (2^-8 for a bf16 C,
whose rounding alone reaches 2^-9), and with the fp32-summation error bound
K 2^-24 S + u_out |ref| + 2^-24, S = sum_k |a b|.
"""
import math

import numpy as np
import pytest

import dense_tiled_gemm_relu_amd as gr
import oracle
import workloads as wl
from tests.helpers import (built_configs, check_close, from_device, fp32_sum_bound, out_tensor,
                           to_device, unit_roundoff)

pytestmark = pytest.mark.gpu

# the two-region grids (256x256 tiles over the first tile columns, narrower
# tiles over the rest), forced here with GEMM_RELU_SPLIT_COLS=1 (one 256-wide
# column first): four waves with 256x192 tiles, or eight waves with 128x384
# ones (GEMM_RELU_FORCE_CONFIG names the eight-wave 256x256 tile)
SPLIT = "d256x256x32_s4_i16+d256x192x32_s4_i16"
SPLIT8 = "d256x256x32_s4_i16w8+d128x384x32_s4_i16w8"
SPLITS = {SPLIT: None, SPLIT8: "d256x256x32_s4_i16w8"}
# built for 16-bit inputs with B stored (N,K) only
NK_ONLY = {"d256x192x32_s4_i16", "d128x384x32_s4_i16w8", SPLIT, SPLIT8}
# the persistent 16x16-block stream: whole 256x256 tiles (M, N >= 256), K a
# multiple of 32 with at least 4 steps
PSTREAM = "d256x256x32_s4_i16p"
DIRECT = built_configs(["d256x256x64_s2", "d256x256x32_s4", "d256x256x32_s5", "d256x256x32_s4_i",
                        "d256x256x64_s2_16", "d256x256x32_s4_i16", "d256x256x32_s4_ip",
                        "d256x256x32_s4_isk", "d256x256x32_s4_w8i", "d256x256x32_s5_w8i",
                        "d256x256x64_s2_w8", "d128x128x64_s3", "d64x64x64_s4", "d64x32x128_s4",
                        "d32x64x128_s4", "d256x192x32_s4_i16", SPLIT, PSTREAM, "d256x256x32_s4_i16w8",
                        "d128x384x32_s4_i16w8", SPLIT8])
STAGED = ["g128x128x64", "g64x64x64"]
COMBOS = [(i, o) for i in (wl.F16, wl.BF16) for o in (wl.F16, wl.BF16, wl.F32)]


@pytest.fixture(autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    yield


BN_OF = {"d256x256x64_s2": 256, "d256x256x32_s4": 256, "d256x256x32_s5": 256,
         "d256x256x32_s4_i": 256, "d256x256x64_s2_16": 256, "d256x256x32_s4_i16": 256, "d256x256x32_s4_ip": 256,
         "d256x256x32_s4_i16w8": 256,
         "d256x256x32_s4_isk": 256,
         "d256x256x32_s4_w8i": 256, "d256x256x32_s5_w8i": 256,
         "d256x256x64_s2_w8": 256, "d128x128x64_s3": 128, "d64x64x64_s4": 64,
         "d64x32x128_s4": 32, "d32x64x128_s4": 64}


def usable(cfg, N, transB, K=None, in_code=wl.F16):
    """Direct-copy configurations need a full tile of columns of a (K,N) B; the
    stream-K one at least two K steps (32 elements, 64 for 8-bit inputs); the
    256x192 tile and the two-region grid B stored (N,K) (the grid also more
    than one 256-wide column)."""
    if cfg in NK_ONLY and not transB:
        return False
    if cfg in SPLITS and N <= 256:
        return False
    if cfg == PSTREAM and (N < 256 or K is None or K % 32 or K < 128):
        return False
    if cfg == "d256x256x32_s4_isk" and K is not None:
        step = 64 if in_code in (wl.F8E4M3, wl.F8E5M2) else 32
        if -(-K // step) < 2:
            return False
    return cfg not in BN_OF or transB or N >= BN_OF[cfg]


def run(A, B, M, N, K, in_code, out_code, transB, cfg=None, monkeypatch=None, poison=True):
    """Upload, call gemm_relu through the C-ABI, return exact binary64 values."""
    import torch
    if cfg in SPLITS:
        monkeypatch.setenv("GEMM_RELU_SPLIT_COLS", "1")
    if cfg is not None:
        force = SPLITS.get(cfg, cfg)
        if force is not None:
            monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", force)
        Ad, Bd = to_device(A, in_code, (M, K)), to_device(B, in_code, wl.b_shape(M, N, K, transB))
        Cd = out_tensor(M, N, out_code, float("nan") if poison else 0.0)
        assert gr.gemm_relu_plan(Ad, Bd, Cd, M, N, K, in_code, out_code, transB) == cfg
    else:
        Ad, Bd = to_device(A, in_code, (M, K)), to_device(B, in_code, wl.b_shape(M, N, K, transB))
        Cd = out_tensor(M, N, out_code, float("nan") if poison else 0.0)
    gr.gemm_relu(Ad, Bd, Cd, M, N, K, in_code, out_code, transB)
    torch.cuda.synchronize()
    return from_device(Cd)


def int_inputs(M, N, K, in_code, transB, seed, out_code):
    # bf16 holds every integer only up to 256: keep |C| small there
    lo, hi = (-1, 1) if out_code == wl.BF16 else (-2, 2)
    A = wl.integers((M, K), seed, in_code, lo, hi)
    B = wl.integers(wl.b_shape(M, N, K, transB), seed + 1, in_code, lo, hi)
    return A, B


def exact_limit(out_code):
    return {wl.F16: 2048.0, wl.BF16: 256.0, wl.F32: 2.0 ** 24}[out_code]


# --------------------------------------------------- every configuration
@pytest.mark.parametrize("cfg", DIRECT + STAGED)
@pytest.mark.parametrize("in_code,out_code", COMBOS)
@pytest.mark.parametrize("transB", [0, 1])
@pytest.mark.parametrize("shape", [(264, 520, 200), (301, 517, 203)], ids=["k8", "ragged"])
def test_configs_integer_bitexact(cfg, in_code, out_code, transB, shape, monkeypatch):
    if cfg in NK_ONLY and not transB:
        pytest.skip("built for B stored (N,K) only")
    if cfg == PSTREAM:
        pytest.skip("the persistent stream needs K a multiple of 32 (its own tests below)")
    # several tiles in every direction plus M, N and K tails (K % BK != 0 in
    # both shapes; the ragged one has odd row lengths, so 2-byte-aligned rows)
    M, N, K = shape
    A, B = int_inputs(M, N, K, in_code, transB, 100, out_code)
    ref = oracle.gemm_relu_ref(A, B, M, N, K, in_code, transB)
    assert np.abs(ref).max() < exact_limit(out_code)
    got = run(A, B, M, N, K, in_code, out_code, transB, cfg, monkeypatch)
    assert np.array_equal(got, ref)
    assert not np.any(np.signbit(got))


@pytest.mark.parametrize("cfg", DIRECT + STAGED)
@pytest.mark.parametrize("in_code,out_code", [(wl.F16, wl.F16), (wl.BF16, wl.F32),
                                              (wl.F16, wl.F32), (wl.BF16, wl.BF16)])
@pytest.mark.parametrize("transB", [0, 1])
def test_configs_uniform_tolerance(cfg, in_code, out_code, transB, monkeypatch):
    if cfg in NK_ONLY and not transB:
        pytest.skip("built for B stored (N,K) only")
    if cfg == PSTREAM:
        pytest.skip("the persistent stream needs K a multiple of 32 (its own tests below)")
    M, N, K = (331, 263, 461)
    A, B = wl.make_inputs(M, N, K, in_code, transB, "uniform", 200)
    got = run(A, B, M, N, K, in_code, out_code, transB, cfg, monkeypatch)
    ref = oracle.gemm_relu_ref(A, B, M, N, K, in_code, transB)
    check_close(got, ref, K, out_code)
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    _, absum = oracle.gemm_relu_ref_at(A, B, rows.ravel(), cols.ravel(), M, N, K, in_code, transB)
    bound = fp32_sum_bound(absum.reshape(M, N), ref, K, unit_roundoff(out_code))
    assert np.all(np.abs(got - ref) <= bound)


# ------------------------------------------------ coded mapping (index bugs)
@pytest.mark.parametrize("cfg", DIRECT + STAGED)
@pytest.mark.parametrize("transB", [0, 1])
def test_coded_mapping(cfg, transB, monkeypatch):
    """A selects one row of B per output row (A[i][pi(i)] = 1), and B's entries
    encode their position, so every output element names its source."""
    if cfg in NK_ONLY and not transB:
        pytest.skip("built for B stored (N,K) only")
    if cfg == PSTREAM:
        pytest.skip("the persistent stream needs K a multiple of 32 (its own tests below)")
    M, N, K = (203, 333, 269)
    rng = np.random.default_rng(3)
    pi = rng.permutation(K)[:M]
    a = np.zeros((M, K))
    a[np.arange(M), pi] = 1.0
    k = np.arange(K)[:, None]
    j = np.arange(N)[None, :]
    bkn = ((131 * k + 7 * j) % 5 - 2).astype(np.float64)
    b = bkn.T if transB else bkn
    A, B = wl.encode(a, wl.F16), wl.encode(b, wl.F16)
    got = run(A, B, M, N, K, wl.F16, wl.F16, transB, cfg, monkeypatch)
    assert np.array_equal(got, np.maximum(bkn[pi, :], 0.0))


# ------------------------------------------- the persistent 16x16 stream
# Each workgroup runs the K steps of several tiles as one stream through the
# stage ring (the next tile's first steps fetched during the current tile's
# last ones); GEMM_RELU_PERSISTENT_GRID makes small problems give every
# workgroup several tiles.  Shapes: one tile, whole tiles, moved-back last
# tile row and column (M, N not multiples of 256), K of exactly one ring (4
# steps) and long K.
PSTREAM_SHAPES = [(256, 256, 128), (512, 768, 256), (777, 530, 160), (520, 1000, 1024), (300, 260, 4096)]
need_pstream = pytest.mark.skipif(not built_configs([PSTREAM]),
                                  reason="the persistent stream is a comparison configuration, not in this build")


@need_pstream
@pytest.mark.parametrize("M,N,K", PSTREAM_SHAPES)
@pytest.mark.parametrize("grid", [1, 3, 8, 0])
@pytest.mark.parametrize("transB", [0, 1])
def test_persistent_stream_integer_bitexact(M, N, K, grid, transB, monkeypatch):
    monkeypatch.setenv("GEMM_RELU_PERSISTENT_GRID", str(grid))
    for in_code, out_code in ((wl.F16, wl.F16), (wl.BF16, wl.F32), (wl.F16, wl.BF16)):
        A, B = int_inputs(M, N, K, in_code, transB, 1100 + M + K + grid, out_code)
        ref = oracle.gemm_relu_ref(A, B, M, N, K, in_code, transB)
        assert np.abs(ref).max() < exact_limit(out_code)
        got = run(A, B, M, N, K, in_code, out_code, transB, PSTREAM, monkeypatch)
        assert np.array_equal(got, ref)
        assert not np.any(np.signbit(got))


@need_pstream
@pytest.mark.parametrize("transB", [0, 1])
def test_persistent_stream_coded_mapping(transB, monkeypatch):
    """Every output names its source row and column (as test_coded_mapping),
    with three tiles per workgroup and moved-back edge tiles."""
    monkeypatch.setenv("GEMM_RELU_PERSISTENT_GRID", "2")
    M, N, K = (523, 777, 288)
    rng = np.random.default_rng(5)
    pi = rng.permutation(K)[:M] if M <= K else rng.integers(0, K, M)
    a = np.zeros((M, K))
    a[np.arange(M), pi] = 1.0
    k = np.arange(K)[:, None]
    j = np.arange(N)[None, :]
    bkn = ((131 * k + 7 * j) % 5 - 2).astype(np.float64)
    b = bkn.T if transB else bkn
    A, B = wl.encode(a, wl.F16), wl.encode(b, wl.F16)
    got = run(A, B, M, N, K, wl.F16, wl.F16, transB, PSTREAM, monkeypatch)
    assert np.array_equal(got, np.maximum(bkn[pi, :], 0.0))


@need_pstream
@pytest.mark.parametrize("in_code,out_code", [(wl.F16, wl.F16), (wl.BF16, wl.F32)])
@pytest.mark.parametrize("transB", [0, 1])
def test_persistent_stream_uniform_tolerance(in_code, out_code, transB, monkeypatch):
    monkeypatch.setenv("GEMM_RELU_PERSISTENT_GRID", "4")
    M, N, K = (600, 700, 480)
    A, B = wl.make_inputs(M, N, K, in_code, transB, "uniform", 1200)
    got = run(A, B, M, N, K, in_code, out_code, transB, PSTREAM, monkeypatch)
    ref = oracle.gemm_relu_ref(A, B, M, N, K, in_code, transB)
    check_close(got, ref, K, out_code)
    absum = oracle.gemm_absum_matmul(A, B, M, N, K, in_code, transB)
    assert np.all(np.abs(got - ref) <= fp32_sum_bound(absum, ref, K, unit_roundoff(out_code)))


@need_pstream
def test_persistent_stream_repeats_and_guards(monkeypatch):
    """Bit-identical results over calls and grid sizes; C's guard bands untouched."""
    import torch
    M, N, K = (777, 530, 320)
    A, B = wl.make_inputs(M, N, K, wl.F16, 0, "uniform", 1300)
    outs = []
    for grid in (1, 5, 0, 0):
        monkeypatch.setenv("GEMM_RELU_PERSISTENT_GRID", str(grid))
        monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", PSTREAM)
        Ad, Bd = to_device(A, wl.F16, (M, K)), to_device(B, wl.F16, (K, N))
        buf = torch.full((M * N + 2048,), 7.0, dtype=torch.float16, device="cuda")
        C = buf[1024:1024 + M * N].view(M, N)
        assert gr.gemm_relu_plan(Ad, Bd, C, M, N, K, wl.F16, wl.F16, 0) == PSTREAM
        gr.gemm_relu(Ad, Bd, C, M, N, K, wl.F16, wl.F16, 0)
        torch.cuda.synchronize()
        assert torch.all(buf[:1024] == 7.0) and torch.all(buf[1024 + M * N:] == 7.0)
        outs.append(C.clone())
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


# ----------------------------------------------------------- 8-bit inputs
FP8_CONFIGS = built_configs(["d256x256x32_s4_i", "d256x256x32_s4_isk", "d128x128x64_s3",
                             "d64x64x64_s4", "d64x32x128_s4", "d32x64x128_s4", "g128x128x64",
                             "g64x64x64"])
FP8 = [wl.F8E4M3, wl.F8E5M2]


@pytest.mark.parametrize("cfg", FP8_CONFIGS)
@pytest.mark.parametrize("in_code", FP8)
@pytest.mark.parametrize("out_code", [wl.F16, wl.BF16, wl.F32])
@pytest.mark.parametrize("transB", [0, 1])
@pytest.mark.parametrize("shape", [(264, 520, 400), (301, 517, 203)], ids=["k16", "ragged"])
def test_fp8_configs_integer_bitexact(cfg, in_code, out_code, transB, shape, monkeypatch):
    # 8-bit rows of odd length start at every byte offset; K % BK != 0 in both
    M, N, K = shape
    A, B = int_inputs(M, N, K, in_code, transB, 600, out_code)
    ref = oracle.gemm_relu_ref(A, B, M, N, K, in_code, transB)
    assert np.abs(ref).max() < exact_limit(out_code)
    got = run(A, B, M, N, K, in_code, out_code, transB, cfg, monkeypatch)
    assert np.array_equal(got, ref)
    assert not np.any(np.signbit(got))


@pytest.mark.parametrize("cfg", FP8_CONFIGS)
@pytest.mark.parametrize("in_code", FP8)
@pytest.mark.parametrize("transB", [0, 1])
def test_fp8_configs_uniform_tolerance(cfg, in_code, transB, monkeypatch):
    M, N, K = (331, 263, 461)
    A, B = wl.make_inputs(M, N, K, in_code, transB, "uniform", 210)
    got = run(A, B, M, N, K, in_code, wl.F16, transB, cfg, monkeypatch)
    ref = oracle.gemm_relu_ref(A, B, M, N, K, in_code, transB)
    check_close(got, ref, K, wl.F16)
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    _, absum = oracle.gemm_relu_ref_at(A, B, rows.ravel(), cols.ravel(), M, N, K, in_code, transB)
    bound = fp32_sum_bound(absum.reshape(M, N), ref, K, unit_roundoff(wl.F16))
    assert np.all(np.abs(got - ref) <= bound)


@pytest.mark.parametrize("cfg", FP8_CONFIGS)
@pytest.mark.parametrize("transB", [0, 1])
def test_fp8_coded_mapping(cfg, transB, monkeypatch):
    """As test_coded_mapping, with E4M3 operands."""
    M, N, K = (203, 333, 269)
    rng = np.random.default_rng(4)
    pi = rng.permutation(K)[:M]
    a = np.zeros((M, K))
    a[np.arange(M), pi] = 1.0
    k = np.arange(K)[:, None]
    j = np.arange(N)[None, :]
    bkn = ((131 * k + 7 * j) % 5 - 2).astype(np.float64)
    b = bkn.T if transB else bkn
    A, B = wl.encode(a, wl.F8E4M3), wl.encode(b, wl.F8E4M3)
    got = run(A, B, M, N, K, wl.F8E4M3, wl.F16, transB, cfg, monkeypatch)
    assert np.array_equal(got, np.maximum(bkn[pi, :], 0.0))


@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (65, 72, 136), (33, 200, 520), (300, 16, 64),
                                   (70, 300, 24), (257, 263, 1), (5, 259, 37), (129, 264, 200)])
@pytest.mark.parametrize("transB", [0, 1])
@pytest.mark.parametrize("in_code", FP8)
def test_fp8_tail_shapes(M, N, K, transB, in_code):
    A, B = int_inputs(M, N, K, in_code, transB, 700 + M, wl.F32)
    ref = oracle.gemm_relu_ref(A, B, M, N, K, in_code, transB)
    got = run(A, B, M, N, K, in_code, wl.F32, transB)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("off_a,off_b", [(1, 0), (0, 3), (5, 7), (15, 1)])
@pytest.mark.parametrize("transB", [0, 1])
def test_fp8_unaligned_pointers(off_a, off_b, transB):
    """8-bit operands that start 1..15 bytes past an aligned allocation."""
    import torch
    M, N, K = 300, 520, 264
    A, B = int_inputs(M, N, K, wl.F8E4M3, transB, 750, wl.F16)
    Ab = torch.zeros(M * K + 16, dtype=torch.uint8, device="cuda")
    Bb = torch.zeros(K * N + 16, dtype=torch.uint8, device="cuda")
    Ab[off_a:off_a + M * K] = torch.from_numpy(A.reshape(-1)).cuda()
    Bb[off_b:off_b + K * N] = torch.from_numpy(B.reshape(-1)).cuda()
    Cd = out_tensor(M, N, wl.F16)
    gr.gemm_relu(Ab[off_a:], Bb[off_b:], Cd, M, N, K, wl.F8E4M3, wl.F16, transB)
    torch.cuda.synchronize()
    assert np.array_equal(from_device(Cd),
                          oracle.gemm_relu_ref(A, B, M, N, K, wl.F8E4M3, transB))


def test_fp8_matmul_relu_front_end():
    import torch
    M, N, K = 130, 260, 200
    A, B = int_inputs(M, N, K, wl.F8E5M2, 0, 760, wl.F16)
    Ad, Bd = to_device(A, wl.F8E5M2, (M, K)), to_device(B, wl.F8E5M2, (K, N))
    C = gr.matmul_relu(Ad, Bd)
    torch.cuda.synchronize()
    assert C.dtype == torch.float16
    assert np.array_equal(from_device(C), oracle.gemm_relu_ref(A, B, M, N, K, wl.F8E5M2, 0))


# ----------------------------------------------------------- tail sweep
SIZES = [1, 2, 7, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 258]
TAIL_SHAPES = [(SIZES[i], SIZES[(i + 5) % 19], SIZES[(i + 11) % 19]) for i in range(19)] + \
              [(SIZES[(i + 7) % 19], SIZES[i], SIZES[(i + 3) % 19]) for i in range(19)] + \
              [(40, 8, 8), (8, 40, 24), (129, 264, 72), (257, 136, 8), (1, 8, 8)]


@pytest.mark.parametrize("M,N,K", TAIL_SHAPES)
@pytest.mark.parametrize("transB", [0, 1])
def test_tail_sweep_integer(M, N, K, transB):
    A, B = int_inputs(M, N, K, wl.F16, transB, 300 + M + N + K, wl.F16)
    ref = oracle.gemm_relu_ref(A, B, M, N, K, wl.F16, transB)
    got = run(A, B, M, N, K, wl.F16, wl.F16, transB)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("cfg", DIRECT + STAGED)
@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (65, 72, 136), (33, 200, 520), (300, 16, 64),
                                   (70, 300, 24), (257, 263, 1), (5, 259, 37)])
def test_tail_shapes_every_config(cfg, M, N, K, monkeypatch):
    tb = 1 if cfg in NK_ONLY else 0
    if cfg == PSTREAM:
        pytest.skip("the persistent stream needs M, N >= 256 (its own tests below)")
    if not usable(cfg, N, tb, K, wl.BF16):
        pytest.skip("needs a full tile of B columns (stream-K: two K steps; two-region grid: "
                    "two tile columns)")
    A, B = int_inputs(M, N, K, wl.BF16, tb, 400 + M, wl.F32)
    ref = oracle.gemm_relu_ref(A, B, M, N, K, wl.BF16, tb)
    got = run(A, B, M, N, K, wl.BF16, wl.F32, tb, cfg, monkeypatch)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("transB", [0, 1])
def test_k_beyond_32_bit_copy_offsets(transB):
    """K past 2^22: a tile's rows of A span more than 2^32 bytes of copy
    offsets, so the plan takes the register-staged tile (64-bit addressing);
    every output bit-exact (elements in {-1, 0, 1}: every partial sum below
    2^24, exact in fp32)."""
    M, N, K = 64, 64, (1 << 22) + 72
    A = wl.integers((M, K), 1600 + transB, wl.F16, -1, 1)
    B = wl.integers(wl.b_shape(M, N, K, transB), 1700 + transB, wl.F16, -1, 1)
    Ad, Bd = to_device(A, wl.F16, (M, K)), to_device(B, wl.F16, wl.b_shape(M, N, K, transB))
    Cd = out_tensor(M, N, wl.F32, float("nan"))
    assert gr.gemm_relu_plan(Ad, Bd, Cd, M, N, K, wl.F16, wl.F32, transB).startswith("g")
    gr.gemm_relu(Ad, Bd, Cd, M, N, K, wl.F16, wl.F32, transB)
    import torch
    torch.cuda.synchronize()
    got = from_device(Cd)
    del Ad, Bd
    assert np.array_equal(got, oracle.gemm_relu_ref_matmul(A, B, M, N, K, wl.F16, transB))


@pytest.mark.parametrize("off_a,off_b,off_c", [(1, 0, 0), (0, 1, 0), (0, 0, 1), (1, 3, 5)])
@pytest.mark.parametrize("transB", [0, 1])
def test_unaligned_pointers(off_a, off_b, off_c, transB):
    """Operands that start 2, 6 or 10 bytes past an aligned allocation."""
    import torch
    M, N, K = 300, 520, 264
    A, B = int_inputs(M, N, K, wl.F16, transB, 450, wl.F16)
    Ab = torch.zeros(M * K + 8, dtype=torch.int16, device="cuda")
    Bb = torch.zeros(K * N + 8, dtype=torch.int16, device="cuda")
    Cb = torch.full((M * N + 8,), float("nan"), dtype=torch.float16, device="cuda")
    Ab[off_a:off_a + M * K] = torch.from_numpy(A.reshape(-1).view(np.int16)).cuda()
    Bb[off_b:off_b + K * N] = torch.from_numpy(B.reshape(-1).view(np.int16)).cuda()
    Ad, Bd, Cd = Ab[off_a:], Bb[off_b:], Cb[off_c:off_c + M * N]
    gr.gemm_relu(Ad, Bd, Cd, M, N, K, wl.F16, wl.F16, transB)
    torch.cuda.synchronize()
    got = from_device(Cd.view(M, N))
    assert np.array_equal(got, oracle.gemm_relu_ref(A, B, M, N, K, wl.F16, transB))
    assert torch.isnan(Cb[:off_c]).all() and torch.isnan(Cb[off_c + M * N:]).all()


# --------------------------------------------------------- degenerate sizes
@pytest.mark.parametrize("M,N,K", [(64, 64, 0), (37, 19, 0)])
@pytest.mark.parametrize("out_code", [wl.F16, wl.F32])
def test_zero_k_gives_positive_zeros(M, N, K, out_code):
    got = run(np.zeros(0, np.uint16), np.zeros(0, np.uint16), M, N, K, wl.F16, out_code, 0)
    assert np.all(got == 0.0) and not np.any(np.signbit(got))


def test_empty_output_untouched():
    import torch
    C = torch.full((4, 4), 7.0, dtype=torch.float16, device="cuda")
    A = torch.ones((0, 8), dtype=torch.float16, device="cuda")
    B = torch.ones((8, 4), dtype=torch.float16, device="cuda")
    gr.gemm_relu(A, B, C, 0, 4, 8, wl.F16, wl.F16, 0)
    torch.cuda.synchronize()
    assert torch.all(C == 7.0)


# ------------------------------------------------------------ properties
def test_determinism_and_guard_bands():
    import torch
    M, N, K = 520, 776, 1032
    A, B = wl.make_inputs(M, N, K, wl.F16, 0, "uniform", 500)
    Ad, Bd = to_device(A, wl.F16, (M, K)), to_device(B, wl.F16, (K, N))
    guard = 4096
    buf = torch.full((guard + M * N + guard,), float("nan"), dtype=torch.float16, device="cuda")
    C = buf[guard:guard + M * N].view(M, N)
    gr.gemm_relu(Ad, Bd, C, M, N, K, wl.F16, wl.F16, 0)
    first = C.clone()
    for _ in range(3):
        gr.gemm_relu(Ad, Bd, C, M, N, K, wl.F16, wl.F16, 0)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), C.view(torch.int16))
    assert not torch.isnan(C).any()
    assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + M * N:]).all()


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (301, 517, 203)])
def test_transB_matches_row_major_B(M, N, K):
    A, B = int_inputs(M, N, K, wl.F16, 0, 600, wl.F16)
    Bt = np.ascontiguousarray(B.reshape(K, N).T)
    g0 = run(A, B, M, N, K, wl.F16, wl.F16, 0)
    g1 = run(A, Bt, M, N, K, wl.F16, wl.F16, 1)
    assert np.array_equal(g0, g1)


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (301, 517, 203)])
def test_relu_pair_reconstructs_the_product(M, N, K):
    A, B = int_inputs(M, N, K, wl.F16, 0, 700, wl.F16)
    negA = A ^ np.uint16(0x8000)
    X = oracle.gemm_relu_ref(A, B, M, N, K, wl.F16, 0, relu=False)
    gp = run(A, B, M, N, K, wl.F16, wl.F16, 0)
    gn = run(negA, B, M, N, K, wl.F16, wl.F16, 0)
    assert np.array_equal(gp - gn, X)


def test_runs_on_the_callers_stream():
    import torch
    M, N, K = 512, 512, 512
    A, B = int_inputs(M, N, K, wl.F16, 0, 800, wl.F16)
    Ad, Bd = to_device(A, wl.F16, (M, K)), to_device(B, wl.F16, (K, N))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        C = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        gr.gemm_relu(Ad, Bd, C, M, N, K, wl.F16, wl.F16, 0)       # current stream = s
    s.synchronize()
    assert np.array_equal(from_device(C), oracle.gemm_relu_ref(A, B, M, N, K, wl.F16, 0))


def test_matmul_relu_front_end():
    import torch
    M, N, K = 192, 320, 128
    A, B = int_inputs(M, N, K, wl.BF16, 1, 900, wl.F32)
    Ad, Bd = to_device(A, wl.BF16, (M, K)), to_device(B, wl.BF16, (N, K))
    C = gr.matmul_relu(Ad, Bd, transB=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(from_device(C), oracle.gemm_relu_ref(A, B, M, N, K, wl.BF16, 1))


# ------------------------------------------- the workloads at full size
@pytest.mark.parametrize("name", [n for n, w in wl.WORKLOADS.items() if not w.get("mx") and not w.get("sparse")])
def test_workload_full_size(name):
    """Each workload at its full size, in the configuration the bench times,
    every output checked: random inputs against the oracle's binary64 loop
    under the contract bound and the fp32-summation bound; integer inputs bit
    for bit against the oracle's binary64 library-matmul form (exact on
    integers)."""
    w = wl.WORKLOADS[name]
    M, N, K, ic, oc, tb = w["M"], w["N"], w["K"], w["in_dtype"], w["out_dtype"], w["transB"]
    A, B = wl.workload_inputs(name)
    got = run(A, B, M, N, K, ic, oc, tb)
    assert not np.any(np.isnan(got)) and np.all(got >= 0)
    ref = oracle.gemm_relu_ref(A, B, M, N, K, ic, tb)
    check_close(got, ref, K, oc)
    absum = oracle.gemm_absum_matmul(A, B, M, N, K, ic, tb)
    assert np.all(np.abs(got - ref) <= fp32_sum_bound(absum, ref, K, unit_roundoff(oc)))
    del ref, absum
    # about half of the outputs of a zero-mean product are clamped to zero
    frac0 = float(np.mean(got == 0.0))
    assert 0.4 < frac0 < 0.6
    del got

    Ai, Bi = wl.workload_inputs(name, int_values=True)
    goti = run(Ai, Bi, M, N, K, ic, oc, tb)
    refi = oracle.gemm_relu_ref_matmul(Ai, Bi, M, N, K, ic, tb)
    assert np.abs(refi).max() < exact_limit(oc)
    assert np.array_equal(goti, refi)
