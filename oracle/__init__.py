"""CPU oracle for the fused GEMM + ReLU — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU product path
(``dense_tiled_gemm_relu_amd``) never imports it, and the two share no code.

The operation (page "TileLang：GPU/NPU 通用算子 DSL", §3.2 GPU minimal example;
§3.3 for the (N,K)-stored B with transpose_B and the fp32 output):

    ref[i, j] = max( sum_k a(i, k) * b(k, j), 0 )

computed in binary64 from the exact values of the inputs: binary16 and
bfloat16, or the OCP 8-bit formats E4M3 and E5M2 (the FP8 GEMM of that page's
§4.1; the pages give it no scale factors, so it is the same definition over the
8-bit values).  Two independent implementations live here:

* ``gemm_relu_ref`` / ``gemm_relu_ref_at`` — a plain C triple loop
  (``oracle.c``) with its own decoders written from the field definitions,
  OpenMP over rows;
* ``gemm_relu_fraction`` — exact rational arithmetic in pure Python
  (``fractions.Fraction``), for tiny shapes only; it decodes through numpy's
  float16, a bit shift for bfloat16 and torch's CPU float8 types, so it shares
  no decoder with the C code.

Inputs are storage patterns (numpy ``uint16`` arrays for the 16-bit types,
``uint8`` for the 8-bit ones); outputs are binary64 numpy arrays.
"""
import ctypes
import os
from fractions import Fraction

import numpy as np

from . import build as _build

F16 = 0
BF16 = 1
F8E4M3 = 3
F8E5M2 = 4
FP8 = (F8E4M3, F8E5M2)

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.oracle_dec_f16.argtypes = [ctypes.c_uint16]
    lib.oracle_dec_f16.restype = ctypes.c_double
    lib.oracle_dec_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_dec_bf16.restype = ctypes.c_double
    lib.oracle_dec_e4m3.argtypes = [ctypes.c_uint8]
    lib.oracle_dec_e4m3.restype = ctypes.c_double
    lib.oracle_dec_e5m2.argtypes = [ctypes.c_uint8]
    lib.oracle_dec_e5m2.restype = ctypes.c_double
    vp = ctypes.c_void_p
    lib.oracle_decode.argtypes = [vp, f64p, i64, ctypes.c_int]
    lib.oracle_decode.restype = None
    lib.oracle_gemm_relu_f64.argtypes = [vp, vp, f64p, i64, i64, i64,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.oracle_gemm_relu_f64.restype = ctypes.c_int
    lib.oracle_gemm_relu_f64_at.argtypes = [vp, vp, i64p, i64p, i64, f64p, f64p,
                                            i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int]
    lib.oracle_gemm_relu_f64_at.restype = ctypes.c_int
    _lib = lib
    return lib


def _bits(x, dtype):
    """Contiguous storage patterns of the input type: uint8 for the 8-bit
    formats, uint16 for the 16-bit ones."""
    x = np.ascontiguousarray(x)
    want = np.uint8 if dtype in FP8 else np.uint16
    if x.dtype != want:
        raise TypeError("oracle inputs of type %d are %s storage patterns, got %s"
                        % (dtype, np.dtype(want).name, x.dtype))
    return x


def _ptr(x, ctype):
    return x.ctypes.data_as(ctypes.POINTER(ctype))


def _vptr(x):
    return ctypes.c_void_p(x.ctypes.data)


def decode(bits, dtype):
    """Exact binary64 values of storage patterns (C decoder)."""
    lib = _load()
    bits = _bits(bits, dtype)
    out = np.empty(bits.shape, dtype=np.float64)
    lib.oracle_decode(_vptr(bits), _ptr(out, ctypes.c_double), bits.size, dtype)
    return out


def gemm_relu_ref(A, B, M, N, K, dtype, transB=0, relu=True, threads=0,
                  return_threads=False):
    """ref = max(A·op(B), 0) in binary64, shape (M, N).

    A holds M*K patterns (row-major (M,K)); B holds K*N patterns, row-major
    (K,N) if transB == 0, (N,K) if transB == 1.
    """
    lib = _load()
    A = _bits(A, dtype).reshape(-1)
    B = _bits(B, dtype).reshape(-1)
    if A.size != M * K or B.size != K * N:
        raise ValueError("operand sizes do not match M, N, K")
    C = np.empty((M, N), dtype=np.float64)
    used = ctypes.c_int(0)
    rc = lib.oracle_gemm_relu_f64(_vptr(A), _vptr(B),
                                  _ptr(C, ctypes.c_double), M, N, K, dtype, int(transB),
                                  1 if relu else 0, threads, ctypes.byref(used))
    if rc != 0:
        raise ValueError("oracle_gemm_relu_f64 failed (%d)" % rc)
    return (C, used.value) if return_threads else C


def gemm_relu_ref_at(A, B, rows, cols, M, N, K, dtype, transB=0, relu=True):
    """The same definition at positions (rows[t], cols[t]).

    Returns (values, absum) where absum[t] = sum_k |a(i,k) b(k,j)|.
    """
    lib = _load()
    A = _bits(A, dtype).reshape(-1)
    B = _bits(B, dtype).reshape(-1)
    if A.size != M * K or B.size != K * N:
        raise ValueError("operand sizes do not match M, N, K")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in shape")
    out = np.empty(rows.shape, dtype=np.float64)
    absum = np.empty(rows.shape, dtype=np.float64)
    rc = lib.oracle_gemm_relu_f64_at(_vptr(A), _vptr(B),
                                     _ptr(rows, ctypes.c_int64), _ptr(cols, ctypes.c_int64),
                                     rows.size, _ptr(out, ctypes.c_double),
                                     _ptr(absum, ctypes.c_double), M, N, K, dtype,
                                     int(transB), 1 if relu else 0)
    if rc != 0:
        raise ValueError("oracle_gemm_relu_f64_at failed (%d)" % rc)
    return out, absum


def _exact(bits, dtype):
    """Exact rational values of storage patterns through numpy or torch's CPU
    float8 types (not the C decoder)."""
    bits = _bits(bits, dtype)
    if dtype == F16:
        vals = bits.view(np.float16).astype(np.float64)
    elif dtype == BF16:
        vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        import torch
        t = torch.from_numpy(bits.reshape(-1).copy())
        fmt = torch.float8_e4m3fn if dtype == F8E4M3 else torch.float8_e5m2
        vals = t.view(fmt).to(torch.float64).numpy()
    return [Fraction(float(v)) for v in vals.reshape(-1)]


def gemm_relu_fraction(A, B, M, N, K, dtype, transB=0, relu=True):
    """Exact rational max(A·op(B), 0) as a nested list of Fractions (tiny shapes)."""
    a = _exact(A, dtype)
    b = _exact(B, dtype)
    out = []
    for i in range(M):
        row = []
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                bk = b[j * K + k] if transB else b[k * N + j]
                s += a[i * K + k] * bk
            row.append(max(s, Fraction(0)) if relu else s)
        out.append(row)
    return out


def gemm_relu_ref_matmul(A, B, M, N, K, dtype, transB=0, relu=True):
    """The same definition with numpy's binary64 matmul as the summation step.

    Operands are decoded by the C decoder; the sum over k is one library
    matrix product in binary64, so for integer-valued inputs (every partial sum
    an integer below 2^53) the result is exact in any summation order.  For
    full-size problems where the triple loop would take minutes.
    """
    A = _bits(A, dtype).reshape(-1)
    B = _bits(B, dtype).reshape(-1)
    if A.size != M * K or B.size != K * N:
        raise ValueError("operand sizes do not match M, N, K")
    a = decode(A, dtype).reshape(M, K)
    b = decode(B, dtype).reshape((N, K) if transB else (K, N))
    x = a @ (b.T if transB else b)
    if not relu:
        return x
    return np.where(x > 0.0, x, 0.0)
