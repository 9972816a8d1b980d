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
* integer variants draw from {lo..hi} and are exact in every input format.
"""
import numpy as np

F16 = 0
BF16 = 1
F32 = 2
F8E4M3 = 3
F8E5M2 = 4
FP8 = (F8E4M3, F8E5M2)
DTYPE_NAMES = {F16: "f16", BF16: "bf16", F32: "f32", F8E4M3: "f8e4m3", F8E5M2: "f8e5m2"}


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
    # the FP8 GEMM of the first page's capability list at the headline shape
    "gemm_relu_f8e4m3_8192": dict(index=7, M=8192, N=8192, K=8192, in_dtype=F8E4M3,
                                  out_dtype=F16, transB=0, dist="uniform"),
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
