"""Seeded synthetic inputs and the workload table for the fused GEMM + ReLU.

This module holds no arithmetic of the method: it only draws numbers and encodes
them as 16-bit or 8-bit storage patterns.  Both the GPU tests and the CPU oracle tests
take their inputs from here, so the two sides see the same bits.

Recipe (the pages fix the shapes and dtypes but no generator):
* numpy ``default_rng(seed)`` (PCG64); seed_A = 1000*i + 1, seed_B = 1000*i + 2
  for workload index i;
* uniform[-1, 1] drawn in binary64, rounded to binary16 by numpy (nearest-even);
* normal(0, sigma) drawn in binary64, rounded to binary32 (nearest-even), then
  to bfloat16 (nearest-even on the upper half);
* 8-bit inputs (OCP E4M3 / E5M2): the same binary64 draws rounded to nearest
  even by torch's CPU float8 conversion (uniform[-1, 1] never reaches either
  format's overflow);
* integer variants draw from {lo..hi} and are exact in every input format;
* block-scaled (MX) inputs: the same binary64 draws, quantised per 32 elements
  along K as the OCP Microscaling recipe does (shared scale 2^(floor(log2
  max|x|) - emax of the element format), elements rounded to nearest even
  with saturation); E2M1 elements are packed two per byte, even k in the low
  nibble.
"""
import numpy as np

F16 = 0
BF16 = 1
F32 = 2
F8E4M3 = 3
F8E5M2 = 4
FP8 = (F8E4M3, F8E5M2)
MX_E4M3 = 5
MX_E5M2 = 6
MX_E2M1 = 7
MX = (MX_E4M3, MX_E5M2, MX_E2M1)
DTYPE_NAMES = {F16: "f16", BF16: "bf16", F32: "f32", F8E4M3: "f8e4m3", F8E5M2: "f8e5m2",
               MX_E4M3: "mxfp8e4m3", MX_E5M2: "mxfp8e5m2", MX_E2M1: "mxfp4"}


def elem_bytes(dtype):
    return 1 if dtype in FP8 else (4 if dtype == F32 else 2)


def f32_to_bf16_bits(x):
    """binary32 values -> bfloat16 patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def encode(values, dtype):
    """binary64 values -> storage patterns of ``dtype`` (nearest-even): uint16
    for the 16-bit types, uint8 for the 8-bit ones."""
    values = np.asarray(values, dtype=np.float64)
    if dtype == F16:
        return values.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        return f32_to_bf16_bits(values.astype(np.float32))
    if dtype in FP8:
        import torch
        fmt = torch.float8_e4m3fn if dtype == F8E4M3 else torch.float8_e5m2
        t = torch.from_numpy(np.ascontiguousarray(values)).to(fmt)
        return t.view(torch.uint8).numpy().copy()
    raise ValueError("input dtypes are f16, bf16, f8e4m3 and f8e5m2")


def uniform(shape, seed, dtype=F16, lo=-1.0, hi=1.0):
    rng = np.random.default_rng(seed)
    return encode(rng.uniform(lo, hi, size=shape), dtype)


def normal(shape, seed, sigma, dtype=BF16):
    rng = np.random.default_rng(seed)
    return encode(rng.normal(0.0, sigma, size=shape), dtype)


def integers(shape, seed, dtype=F16, lo=-2, hi=2):
    rng = np.random.default_rng(seed)
    return encode(rng.integers(lo, hi + 1, size=shape).astype(np.float64), dtype)


def seeds(index):
    return 1000 * index + 1, 1000 * index + 2


# The workloads: shapes and dtypes of the pages' running example (fp16 in, fp32
# accumulate, fp16 out; bf16 with B stored (N,K) and fp32 out as on the Ascend
# version) at the sizes used for parity and measurement.
WORKLOADS = {
    "gemm_relu_f16_256": dict(index=1, M=256, N=256, K=256, in_dtype=F16, out_dtype=F16,
                              transB=0, dist="uniform"),
    "gemm_relu_f16_4096": dict(index=2, M=4096, N=4096, K=4096, in_dtype=F16, out_dtype=F16,
                               transB=0, dist="uniform"),
    "gemm_relu_f16_8192": dict(index=3, M=8192, N=8192, K=8192, in_dtype=F16, out_dtype=F16,
                               transB=0, dist="uniform"),
    "gemm_relu_bf16_tB_f32_4096x7168x4096": dict(index=4, M=4096, N=7168, K=4096, in_dtype=BF16,
                                                 out_dtype=F32, transB=1, dist="normal"),
    "gemm_relu_f16_4097x3001x5003": dict(index=5, M=4097, N=3001, K=5003, in_dtype=F16,
                                         out_dtype=F16, transB=0, dist="uniform"),
    "gemm_relu_f16_64x8192x8192": dict(index=6, M=64, N=8192, K=8192, in_dtype=F16,
                                       out_dtype=F16, transB=0, dist="uniform"),
    # the FP8 GEMM of the capability list of page "TileLang：GPU/NPU 通用算子 DSL"
    # (§4.1), at the headline shape
    "gemm_relu_f8e4m3_8192": dict(index=7, M=8192, N=8192, K=8192, in_dtype=F8E4M3,
                                  out_dtype=F16, transB=0, dist="uniform"),
    # block-scaled (gemm_relu_mx): the MXFP4 / MXFP8 of the same list, B stored (N, K)
    "gemm_relu_mxfp4_8192": dict(index=8, M=8192, N=8192, K=8192, in_dtype=MX_E2M1,
                                 out_dtype=F16, transB=1, dist="uniform", mx=True),
    "gemm_relu_mxfp8_8192": dict(index=9, M=8192, N=8192, K=8192, in_dtype=MX_E4M3,
                                 out_dtype=F16, transB=1, dist="uniform", mx=True),
    # 2:4 sparse A (gemm_relu_sp): the T.gemm_sp of the same list, B (K, N)
    "gemm_relu_sp_f16_8192": dict(index=10, M=8192, N=8192, K=8192, in_dtype=F16,
                                  out_dtype=F16, transB=0, dist="uniform", sparse=True),
}


def b_shape(M, N, K, transB):
    return (N, K) if transB else (K, N)


def make_inputs(M, N, K, in_dtype, transB, dist, index, int_values=False):
    """(A, B) as uint16 arrays, A (M,K) and B (K,N) or (N,K)."""
    sa, sb = seeds(index)
    bshape = b_shape(M, N, K, transB)
    if int_values:
        return integers((M, K), sa, in_dtype), integers(bshape, sb, in_dtype)
    if dist == "uniform":
        return uniform((M, K), sa, in_dtype), uniform(bshape, sb, in_dtype)
    if dist == "normal":
        sigma = 1.0 / np.sqrt(K)
        return normal((M, K), sa, sigma, in_dtype), normal(bshape, sb, sigma, in_dtype)
    raise ValueError(dist)


def workload_inputs(name, int_values=False):
    w = WORKLOADS[name]
    return make_inputs(w["M"], w["N"], w["K"], w["in_dtype"], w["transB"], w["dist"],
                       w["index"], int_values)


# ----------------------------------------------- block-scaled (MX) inputs
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_MX_EMAX = {MX_E4M3: 8, MX_E5M2: 15, MX_E2M1: 2}


def e2m1_codes(values):
    """binary64 values -> E2M1 nibbles, nearest (ties to the even code), saturating at 6."""
    v = np.asarray(values, dtype=np.float64)
    mag = np.minimum(np.abs(v), 6.0)
    d = np.abs(mag[..., None] - _E2M1_MAG)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # among equally near codes take the even one (fraction bit 0)
    even = cand & (np.arange(8) % 2 == 0)
    code = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    return (code | np.where(np.signbit(v) & (code != 0), 8, 0)).astype(np.uint8)


def pack_e2m1(codes):
    """(rows, K) nibbles -> (rows, K/2) bytes, even k in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def mx_quantize(values, fmt):
    """(rows, K) binary64 values, K % 32 == 0 -> (elements, scales) as uint8
    arrays: elements (rows, K) (E4M3 / E5M2) or (rows, K/2) (packed E2M1),
    scales (rows, K/32) E8M0."""
    v = np.asarray(values, dtype=np.float64)
    rows, K = v.shape
    blocks = v.reshape(rows, K // 32, 32)
    amax = np.abs(blocks).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))), 0.0)
    shared = np.clip(e - _MX_EMAX[fmt], -127, 127).astype(np.int64)
    scales = (shared + 127).astype(np.uint8)
    x = blocks / np.ldexp(1.0, shared)[..., None]
    if fmt == MX_E2M1:
        elems = pack_e2m1(e2m1_codes(x).reshape(rows, K))
    else:
        import torch
        tfmt = torch.float8_e4m3fn if fmt == MX_E4M3 else torch.float8_e5m2
        lim = 448.0 if fmt == MX_E4M3 else 57344.0
        t = torch.from_numpy(np.clip(x, -lim, lim).reshape(rows, K)).to(tfmt)
        elems = t.view(torch.uint8).numpy().copy()
    return elems, scales


def mx_inputs(M, N, K, fmt, index, dist="uniform", int_values=False):
    """(A, SA, B, SB) for a block-scaled product: A (M, K), B stored (N, K)."""
    sa, sb = seeds(index)
    ra, rb = np.random.default_rng(sa), np.random.default_rng(sb)
    if int_values:
        # small integers with unit scales (E8M0 127): exact in every element format
        a = ra.integers(-2, 3, size=(M, K)).astype(np.float64)
        b = rb.integers(-2, 3, size=(N, K)).astype(np.float64)
        qa = (pack_e2m1(e2m1_codes(a)) if fmt == MX_E2M1 else encode(a, F8E4M3 if fmt == MX_E4M3 else F8E5M2))
        qb = (pack_e2m1(e2m1_codes(b)) if fmt == MX_E2M1 else encode(b, F8E4M3 if fmt == MX_E4M3 else F8E5M2))
        return (qa, np.full((M, K // 32), 127, np.uint8), qb, np.full((N, K // 32), 127, np.uint8))
    a = ra.uniform(-1.0, 1.0, size=(M, K))
    b = rb.uniform(-1.0, 1.0, size=(N, K))
    qa, xa = mx_quantize(a, fmt)
    qb, xb = mx_quantize(b, fmt)
    return qa, xa, qb, xb


# ------------------------------------------------------- 2:4 sparse A
# The six position pairs (p0 < p1) a group of four can keep.
SP_PAIRS = [(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)]


def sp_meta_bytes(M, K):
    """Bytes of the metadata E of an (M, K) sparse A: ceil(K/64) blocks of M x 8."""
    return ((K + 63) // 64) * M * 8


def sp_pack(positions, M, K):
    """positions: (M, K/4, 2) int array of (p0, p1) per group -> E bytes
    (blocked by 64 columns of K; group q of row i in nibble q % 2 of byte
    (q % 16) / 2 of row i's 8 bytes in block q / 16; nibble = p0 | p1 << 2)."""
    E = np.zeros(sp_meta_bytes(M, K), dtype=np.uint8)
    pos = np.asarray(positions, dtype=np.int64)
    nib = (pos[..., 0] | (pos[..., 1] << 2)).astype(np.uint8)        # (M, K/4)
    for q in range(K // 4):
        idx = (q // 16) * M * 8 + np.arange(M) * 8 + (q % 16) // 2
        E[idx] |= (nib[:, q] << (4 * (q % 2))).astype(np.uint8)
    return E


def sp_random(M, K, rng, int_values=False):
    """A random 2:4 sparse (M, K) matrix: per group of four, a uniformly chosen
    position pair; values uniform[-1, 1] (or integers in [-3, 3]) in binary64.
    Returns (values (M, K/2), positions (M, K/4, 2), dense (M, K))."""
    choice = rng.integers(0, len(SP_PAIRS), size=(M, K // 4))
    positions = np.asarray(SP_PAIRS, dtype=np.int64)[choice]
    if int_values:
        vals = rng.integers(-3, 4, size=(M, K // 2)).astype(np.float64)
    else:
        vals = rng.uniform(-1.0, 1.0, size=(M, K // 2))
    dense = np.zeros((M, K))
    rows = np.arange(M)[:, None]
    groups = np.arange(K // 4)[None, :]
    dense[rows, 4 * groups + positions[..., 0]] = vals[:, 0::2]
    dense[rows, 4 * groups + positions[..., 1]] = vals[:, 1::2]
    return vals, positions, dense


def sp_inputs(M, N, K, in_dtype, transB, index, int_values=False):
    """(As, E, B) storage for a 2:4 sparse A (values rounded to the input type
    after the draw) and a dense B of the layout transB."""
    sa, sb = seeds(index)
    ra, rb = np.random.default_rng(sa), np.random.default_rng(sb)
    vals, positions, _ = sp_random(M, K, ra, int_values)
    if int_values:
        b = rb.integers(-3, 4, size=b_shape(M, N, K, transB)).astype(np.float64)
    else:
        b = rb.uniform(-1.0, 1.0, size=b_shape(M, N, K, transB))
    return encode(vals, in_dtype), sp_pack(positions, M, K), encode(b, in_dtype)
