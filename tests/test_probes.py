"""gfx950 lane layouts the kernel relies on, checked on the device.

Each probe runs one wave on tiny in-bounds buffers through the same helpers the
GEMM kernel uses (MFMA wrapper, LDS transpose read, direct global->LDS copy).
"""
import ctypes

import numpy as np
import pytest

import dense_tiled_gemm_relu_amd as gr
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probe():
    import torch
    assert torch.cuda.is_available()
    lib = ctypes.CDLL(gr.PROBE_LIB_PATH)
    for name in ("probe_mfma_32x32x16", "probe_mfma_16x16x32", "probe_tr16", "probe_dma16",
                 "probe_unaligned16"):
        getattr(lib, name).restype = ctypes.c_int
    lib.probe_mfma_32x32x16.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int]
    lib.probe_mfma_16x16x32.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int]
    lib.probe_tr16.argtypes = [ctypes.c_void_p] * 3
    lib.probe_dma16.argtypes = [ctypes.c_void_p] * 3
    lib.probe_unaligned16.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_uint, ctypes.c_void_p]
    return lib


def _dev(arr):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
def test_mfma_32x32x16_layout(probe, dtype):
    import torch
    rng = np.random.default_rng(7)
    x = rng.integers(-3, 4, size=(32, 16)).astype(np.float64)
    y = rng.integers(-3, 4, size=(16, 32)).astype(np.float64)
    X = _dev(wl.encode(x, dtype).view(np.int16))
    Y = _dev(wl.encode(y, dtype).view(np.int16))
    D = torch.zeros((32, 32), dtype=torch.float32, device="cuda")
    assert probe.probe_mfma_32x32x16(X.data_ptr(), Y.data_ptr(), D.data_ptr(), dtype) == 0
    assert np.array_equal(D.cpu().numpy().astype(np.float64), x @ y)


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
def test_mfma_16x16x32_layout(probe, dtype):
    """Lane l feeds row/column l % 16 with k group l / 16 (8 consecutive k) and
    owns D[4 (l / 16) + r][l % 16] in result register r."""
    import torch
    rng = np.random.default_rng(8)
    x = rng.integers(-3, 4, size=(16, 32)).astype(np.float64)
    y = rng.integers(-3, 4, size=(32, 16)).astype(np.float64)
    X = _dev(wl.encode(x, dtype).view(np.int16))
    Y = _dev(wl.encode(y, dtype).view(np.int16))
    D = torch.zeros((16, 16), dtype=torch.float32, device="cuda")
    assert probe.probe_mfma_16x16x32(X.data_ptr(), Y.data_ptr(), D.data_ptr(), dtype) == 0
    assert np.array_equal(D.cpu().numpy().astype(np.float64), x @ y)


def test_lds_transpose_read(probe):
    """16 lanes read a 4 x 16 block, 8 bytes each (lane q: row q // 4, columns
    4 (q % 4) .. +3); lane i then holds column i, rows 0..3."""
    import torch
    src = np.arange(4096, dtype=np.uint16)           # LDS viewed as 16 rows x 256
    off = np.zeros(64, dtype=np.uint32)
    want = np.zeros((64, 4), dtype=np.uint16)
    for h in range(4):
        r0, c0 = 4 * h, 16 * h + 8 * (h % 2)
        for q in range(16):
            off[16 * h + q] = ((r0 + q // 4) * 256 + c0 + 4 * (q % 4)) * 2
            for e in range(4):
                want[16 * h + q, e] = (r0 + e) * 256 + c0 + q
    assert off.max() + 8 <= 8192 and np.all(off % 8 == 0)
    out = torch.zeros(256, dtype=torch.int16, device="cuda")
    src_d, off_d = _dev(src.view(np.int16)), _dev(off.view(np.int32))   # alive through the call
    assert probe.probe_tr16(src_d.data_ptr(), off_d.data_ptr(), out.data_ptr()) == 0
    got = out.cpu().numpy().view(np.uint16).reshape(64, 4)
    assert np.array_equal(got, want)


def test_direct_global_to_lds_copy(probe):
    """Lane l's 16 bytes land at LDS offset 16 l whatever global chunk it fetched."""
    import torch
    src = np.arange(512, dtype=np.uint16)
    perm = ((np.arange(64) * 37 + 5) % 64).astype(np.uint32)
    out = torch.zeros(512, dtype=torch.int16, device="cuda")
    src_d, perm_d = _dev(src.view(np.int16)), _dev(perm.view(np.int32))
    assert probe.probe_dma16(src_d.data_ptr(), perm_d.data_ptr(), out.data_ptr()) == 0
    got = out.cpu().numpy().view(np.uint16).reshape(64, 8)
    assert np.array_equal(got, src.reshape(64, 8)[perm])


def test_unaligned_16_byte_loads(probe):
    """16-byte direct copies and vector loads from 2-byte-aligned addresses
    (rows of an odd-length fp16 matrix) return the 8 elements that start there."""
    import torch
    n = 4096
    src = np.arange(n, dtype=np.uint16) * np.uint16(7) + np.uint16(3)
    rng = np.random.default_rng(11)
    off = rng.integers(0, n - 8, size=64).astype(np.uint32)
    off[:8] = [1, 3, 5, 7, 9, 2, 4, 6]                    # every residue mod 8
    out = torch.zeros(1024, dtype=torch.int16, device="cuda")
    src_d, off_d = _dev(src.view(np.int16)), _dev(off.view(np.int32))
    assert probe.probe_unaligned16(src_d.data_ptr(), off_d.data_ptr(), n, out.data_ptr()) == 0
    got = out.cpu().numpy().view(np.uint16).reshape(2, 64, 8)
    want = np.stack([src[o:o + 8] for o in off])
    assert np.array_equal(got[1], want), "plain vector load"
    assert np.array_equal(got[0], want), "direct global->LDS copy"


@pytest.mark.parametrize("kind,opb,cycles", [(0, 16, 32), (1, 32, 64), (2, 16, 32), (3, 32, 64),
                                              (4, 32, 32), (5, 16, 32)],
                         ids=["f16", "e4m3", "mx_e2m1", "mx_e4m3", "sparse_f16", "f16_16x16"])
def test_mfma_rate_probe(probe, kind, opb, cycles):
    """The MFMA-only diagnostic (random operands, no memory traffic) runs, issues
    one 32x32x16 fp16 MFMA per 32 shader cycles (one 32x32x64 E4M3 MFMA per
    64, two 16x16x32 fp16 MFMAs per 32) per SIMD, and keeps its accumulators
    finite; size errors and unknown kinds are rejected before launch."""
    import torch
    lib = probe
    lib.probe_mfma_rate.restype = ctypes.c_int
    lib.probe_mfma_rate.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p]
    blocks, steps = 256, 256
    if kind == 2:                                        # random E2M1 nibble pairs
        src = torch.randint(0, 256, (blocks * 8 * 256 * opb,), dtype=torch.uint8, device="cuda")
    else:
        per_lane = opb // 2 if kind in (0, 4, 5) else opb  # elements per operand per lane
        src = torch.empty(blocks * 8 * 256 * per_lane, dtype=torch.float32, device="cuda")
        src = src.uniform_(-1, 1).to(torch.float16 if kind in (0, 4, 5) else torch.float8_e4m3fn)
    nbytes = src.numel() * src.element_size()
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    ticks = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert lib.probe_mfma_rate(src.data_ptr(), nbytes - 1, out.data_ptr(),
                               ticks.data_ptr(), blocks, steps, kind, st) == -1
    assert lib.probe_mfma_rate(src.data_ptr(), nbytes, out.data_ptr(),
                               ticks.data_ptr(), blocks, steps, 6, st) == -1
    assert lib.probe_mfma_rate(src.data_ptr(), nbytes, out.data_ptr(),
                               ticks.data_ptr(), blocks, steps, kind, st) == 0
    torch.cuda.synchronize()
    cyc = ticks.view(blocks, 2)[:, 0].double().mean().item() / (steps * 32)
    assert cycles - 0.1 <= cyc <= cycles * 1.25, cyc
    assert torch.isfinite(out).all()


# ---------------------------------------------------------- 8-bit data paths
def _fp8_lib():
    lib = ctypes.CDLL(gr.PROBE_LIB_PATH)
    for n in ("probe_mfma_f8_raw", "probe_tr8_raw", "probe_unaligned8"):
        getattr(lib, n).restype = ctypes.c_int
    lib.probe_mfma_f8_raw.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int]
    lib.probe_tr8_raw.argtypes = [ctypes.c_void_p] * 3
    lib.probe_unaligned8.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint,
                                     ctypes.c_void_p]
    return lib


@pytest.mark.parametrize("dtype", [wl.F8E4M3, wl.F8E5M2])
def test_mfma_32x32x64_f8_layout(dtype):
    """v_mfma_f32_32x32x64_f8f6f4 without block scales: lane l feeds row/column
    l % 32 with the 32 bytes of k-group l / 32 (byte e of an A lane meets byte
    e of the B lane of the same group), and owns D[8 (r/4) + 4 (l/32) + r%4][l%32]
    in result register r — the layout of the 16-bit MFMA the kernel uses."""
    import torch
    lib = _fp8_lib()
    rng = np.random.default_rng(21 + dtype)
    av = rng.integers(-3, 4, size=(64, 32)).astype(np.float64)
    bv = rng.integers(-3, 4, size=(64, 32)).astype(np.float64)
    ab, bb = _dev(wl.encode(av, dtype)), _dev(wl.encode(bv, dtype))
    d = torch.zeros(64 * 16, dtype=torch.float32, device="cuda")
    fmt = 0 if dtype == wl.F8E4M3 else 1
    assert lib.probe_mfma_f8_raw(ab.data_ptr(), bb.data_ptr(), d.data_ptr(), fmt) == 0
    X = np.zeros((32, 64))
    Y = np.zeros((64, 32))
    for l in range(64):
        X[l % 32, 32 * (l // 32):32 * (l // 32) + 32] = av[l]
        Y[32 * (l // 32):32 * (l // 32) + 32, l % 32] = bv[l]
    D = X @ Y
    want = np.array([[D[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32] for r in range(16)]
                     for l in range(64)])
    assert np.array_equal(d.cpu().numpy().reshape(64, 16), want)


def test_lds_transpose_read_b8():
    """ds_read_b64_tr_b8: in each 16-lane group, lane i supplies the address of
    8 bytes (row i / 2, columns 8 (i % 2) .. +7 of a 8 x 16 byte block) and
    receives the 8 rows of column i."""
    import torch
    lib = _fp8_lib()
    P = 256
    rng = np.random.default_rng(9)
    M = rng.integers(0, 256, size=(16, P)).astype(np.uint8)
    off = np.zeros(64, dtype=np.uint32)
    col0 = np.zeros(64, dtype=np.int64)
    for l in range(64):
        h, i16 = l // 16, l % 16
        col0[l] = 16 * (h & 1) + 32 * (h >> 1)
        off[l] = (i16 // 2) * P + col0[l] + 8 * (i16 % 2)
    src_d, off_d = _dev(M.reshape(-1)), _dev(off.view(np.int32))
    out = torch.zeros(512, dtype=torch.uint8, device="cuda")
    assert lib.probe_tr8_raw(src_d.data_ptr(), off_d.data_ptr(), out.data_ptr()) == 0
    want = np.stack([M[0:8, col0[l] + l % 16] for l in range(64)])
    assert np.array_equal(out.cpu().numpy().reshape(64, 8), want)


def test_byte_unaligned_16_byte_loads():
    """16-byte direct copies and vector loads from any byte offset (rows of an
    odd-length 8-bit matrix) return the 16 bytes that start there."""
    import torch
    lib = _fp8_lib()
    n = 4096
    src = (np.arange(n) * 7 + 3).astype(np.uint8)
    rng = np.random.default_rng(13)
    off = rng.integers(0, n - 16, size=64).astype(np.uint32)
    off[:16] = np.arange(16) + 1                          # every residue mod 16
    src_d, off_d = _dev(src), _dev(off.view(np.int32))
    out = torch.zeros(2048, dtype=torch.uint8, device="cuda")
    assert lib.probe_unaligned8(src_d.data_ptr(), off_d.data_ptr(), n, out.data_ptr()) == 0
    got = out.cpu().numpy().reshape(2, 64, 16)
    want = np.stack([src[o:o + 16] for o in off])
    assert np.array_equal(got[1], want), "plain vector load"
    assert np.array_equal(got[0], want), "direct global->LDS copy"


# ------------------------------------------------------- 2:4 sparse MFMA
@pytest.mark.parametrize("bf16", [False, True], ids=["f16", "bf16"])
@pytest.mark.parametrize("abid", [0, 1])
def test_smfmac_32x32x32_layout(bf16, abid):
    """v_smfmac_f32_32x32x32: lane 32 g + i of the sparse operand holds the 8
    stored values of groups 4 g .. 4 g + 3 of row i (2 per group, in order);
    its index word holds their positions as nibbles p0 | p1 << 2 in group order
    (bits 0..15, or 16..31 when ABID = 1); lane 32 g + j of the dense operand
    holds k = 8 g .. 8 g + 7 then 16 + 8 g .. 16 + 8 g + 7 of column j; result
    register r of lane l is D[8 (r/4) + 4 (l/32) + r%4][l%32], rows from the
    sparse operand — the layout gemm_sp_relu_kernel.hpp assumes."""
    import torch
    lib = ctypes.CDLL(gr.PROBE_LIB_PATH)
    lib.probe_smfmac_raw.restype = ctypes.c_int
    lib.probe_smfmac_raw.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_int]
    rng = np.random.default_rng(40 + abid + 2 * bf16)
    av = rng.integers(-3, 4, size=(64, 8)).astype(np.float64)
    bv = rng.integers(-3, 4, size=(64, 16)).astype(np.float64)
    pairs = np.asarray(wl.SP_PAIRS)
    pick = rng.integers(0, 6, size=(64, 8))               # 8 groups: both halves of the word
    idx = np.zeros(64, np.uint32)
    for grp in range(8):
        idx |= ((pairs[pick[:, grp], 0] | (pairs[pick[:, grp], 1] << 2)) << (4 * grp)).astype(np.uint32)
    dt = wl.BF16 if bf16 else wl.F16
    a_d = torch.from_numpy(wl.encode(av, dt).view(np.int16)).cuda()
    b_d = torch.from_numpy(wl.encode(bv, dt).view(np.int16)).cuda()
    i_d = torch.from_numpy(idx.view(np.int32)).cuda()
    d = torch.zeros(64 * 16, dtype=torch.float32, device="cuda")
    assert lib.probe_smfmac_raw(a_d.data_ptr(), b_d.data_ptr(), i_d.data_ptr(), d.data_ptr(),
                                1 if bf16 else 0, abid) == 0
    torch.cuda.synchronize()
    A = np.zeros((32, 32))
    Bm = np.zeros((32, 32))
    for lane in range(64):
        i, g = lane % 32, lane // 32
        w = int(idx[lane]) >> (16 * abid)
        for v in range(8):
            pos = (w >> (2 * v)) & 3
            A[i, 16 * g + 4 * (v // 2) + pos] += av[lane, v]
        for e in range(16):
            Bm[8 * g + e if e < 8 else 16 + 8 * g + e - 8, i] = bv[lane, e]
    D = A @ Bm
    want = np.array([[D[8 * (r // 4) + 4 * (lane // 32) + r % 4, lane % 32] for r in range(16)]
                     for lane in range(64)])
    assert np.array_equal(d.cpu().numpy().reshape(64, 16), want)
