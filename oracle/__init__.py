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

Block-scaled (MX) products (the MXFP8 / MXFP4 of that page's §4.1 timeline)
follow the OCP Microscaling definition: ``gemm_relu_mx_ref`` (C) and
``gemm_relu_mx_fraction`` (exact rationals, its own E2M1 table) take A (M, K)
and B stored (N, K) with E8M0 scales per 32 elements along K.

2:4 structured-sparse A (the T.gemm_sp of that page's §4.1 timeline; page
"从 TVM 到 TileLang…", §四, loads the compressed A and its metadata E side by
side): ``gemm_relu_sp_ref`` (C) and ``gemm_relu_sp_fraction`` (exact
rationals, its own metadata reading) decode (As, E) back to the plain A — As
(M, K/2) holds the two stored values of every group of four along K, E their
positions as nibbles p0 | p1 << 2, blocked by 64 columns of K (M x 8 bytes per
block) — and then take the same definition.
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
MX_E4M3 = 5      # MXFP8, E4M3 elements
MX_E5M2 = 6      # MXFP8, E5M2 elements
MX_E2M1 = 7      # MXFP4, E2M1 elements packed two per byte (even k in the low nibble)
MX = (MX_E4M3, MX_E5M2, MX_E2M1)

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("ORACLE_LIB") or _build.LIB      # another build of oracle.c (sanitizers)
    if path == _build.LIB and not os.path.exists(path):
        _build.build()
    lib = ctypes.CDLL(path)
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
    lib.oracle_dec_e2m1.argtypes = [ctypes.c_uint8]
    lib.oracle_dec_e2m1.restype = ctypes.c_double
    lib.oracle_dec_e8m0.argtypes = [ctypes.c_uint8]
    lib.oracle_dec_e8m0.restype = ctypes.c_double
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
    lib.oracle_gemm_relu_mx.argtypes = [vp, vp, vp, vp, i64p, i64p, i64, f64p, f64p,
                                        i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.oracle_gemm_relu_mx.restype = ctypes.c_int
    lib.oracle_gemm_sp_relu.argtypes = [vp, vp, vp, i64p, i64p, i64, f64p, f64p,
                                        i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.oracle_gemm_sp_relu.restype = ctypes.c_int
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


def gemm_absum_matmul(A, B, M, N, K, dtype, transB=0):
    """S[i, j] = sum_k |a(i,k) b(k,j)| for every output, the scale of the
    binary32 summation error bound, with numpy's binary64 matmul of the
    decoded magnitudes as the summation step (a bound's scale, so its own
    rounding does not matter).  For full-size problems."""
    A = _bits(A, dtype).reshape(-1)
    B = _bits(B, dtype).reshape(-1)
    if A.size != M * K or B.size != K * N:
        raise ValueError("operand sizes do not match M, N, K")
    a = np.abs(decode(A, dtype).reshape(M, K))
    b = np.abs(decode(B, dtype).reshape((N, K) if transB else (K, N)))
    return a @ (b.T if transB else b)


# ------------------------------------------------------ block-scaled (MX)
def dec_e2m1(nibble):
    return _load().oracle_dec_e2m1(int(nibble))


def dec_e8m0(e):
    return _load().oracle_dec_e8m0(int(e))


def _mx_check(A, SA, B, SB, M, N, K, fmt):
    if fmt not in MX:
        raise ValueError("MX element format %d" % fmt)
    if K % 32:
        raise ValueError("K must be a multiple of 32 (whole scale blocks)")
    row = K // 2 if fmt == MX_E2M1 else K
    arrs = []
    for x, n in ((A, M * row), (SA, M * (K // 32)), (B, N * row), (SB, N * (K // 32))):
        x = np.ascontiguousarray(x).reshape(-1)
        if x.dtype != np.uint8 or x.size != n:
            raise ValueError("MX operands are uint8 arrays of the documented sizes")
        arrs.append(x)
    return arrs


def gemm_relu_mx_ref(A, SA, B, SB, M, N, K, fmt, relu=True, rows=None, cols=None):
    """Block-scaled max(A·Bᵀ, 0) in binary64: the full (M, N) product, or the
    values and absum at positions (rows[t], cols[t]).  A: M x K elements, B
    stored N x K, SA / SB: (M, K/32) / (N, K/32) E8M0 bytes."""
    lib = _load()
    A, SA, B, SB = _mx_check(A, SA, B, SB, M, N, K, fmt)
    if rows is None:
        out = np.empty((M, N), dtype=np.float64)
        rc = lib.oracle_gemm_relu_mx(_vptr(A), _vptr(SA), _vptr(B), _vptr(SB), None, None, 0,
                                     _ptr(out, ctypes.c_double), None, M, N, K, fmt,
                                     1 if relu else 0)
        if rc != 0:
            raise ValueError("oracle_gemm_relu_mx failed (%d)" % rc)
        return out
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.empty(rows.shape, dtype=np.float64)
    absum = np.empty(rows.shape, dtype=np.float64)
    rc = lib.oracle_gemm_relu_mx(_vptr(A), _vptr(SA), _vptr(B), _vptr(SB),
                                 _ptr(rows, ctypes.c_int64), _ptr(cols, ctypes.c_int64), rows.size,
                                 _ptr(out, ctypes.c_double), _ptr(absum, ctypes.c_double),
                                 M, N, K, fmt, 1 if relu else 0)
    if rc != 0:
        raise ValueError("oracle_gemm_relu_mx failed (%d)" % rc)
    return out, absum


# E2M1 magnitudes as the OCP table lists them (codes 0..7), for the rational twin
_E2M1_TABLE = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
               Fraction(3), Fraction(4), Fraction(6)]


def _mx_elems_exact(row_bytes, K, fmt):
    if fmt == MX_E2M1:
        out = []
        for k in range(K):
            nib = (int(row_bytes[k // 2]) >> (4 * (k % 2))) & 0xF
            v = _E2M1_TABLE[nib & 7]
            out.append(-v if nib & 8 else v)
        return out
    return _exact(np.ascontiguousarray(row_bytes[:K]), F8E4M3 if fmt == MX_E4M3 else F8E5M2)


def gemm_relu_mx_fraction(A, SA, B, SB, M, N, K, fmt, relu=True):
    """Exact rational block-scaled product (tiny shapes): its own E2M1 table,
    torch's float8 types for E4M3 / E5M2, and 2^(e-127) as a Fraction."""
    A, SA, B, SB = _mx_check(A, SA, B, SB, M, N, K, fmt)
    rb = K // 2 if fmt == MX_E2M1 else K
    nb = K // 32
    a = [_mx_elems_exact(A[i * rb:(i + 1) * rb], K, fmt) for i in range(M)]
    b = [_mx_elems_exact(B[j * rb:(j + 1) * rb], K, fmt) for j in range(N)]
    out = []
    for i in range(M):
        row = []
        for j in range(N):
            s = Fraction(0)
            for blk in range(nb):
                xa = Fraction(2) ** (int(SA[i * nb + blk]) - 127)
                xb = Fraction(2) ** (int(SB[j * nb + blk]) - 127)
                for k in range(32 * blk, 32 * blk + 32):
                    s += xa * a[i][k] * xb * b[j][k]
            row.append(max(s, Fraction(0)) if relu else s)
        out.append(row)
    return out


# ------------------------------------------------------- 2:4 sparse A
def sp_meta_bytes(M, K):
    """Size of the metadata array E for an (M, K) sparse A: ceil(K / 64)
    blocks of M x 8 bytes."""
    return ((K + 63) // 64) * M * 8


def _sp_check(As, E, B, M, N, K, dtype, transB):
    if K % 4 != 0:
        raise ValueError("K must be a multiple of 4 (whole groups of four)")
    As = _bits(As, dtype).reshape(-1)
    B = _bits(B, dtype).reshape(-1)
    E = np.ascontiguousarray(E, dtype=np.uint8).reshape(-1)
    if As.size != M * (K // 2) or B.size != K * N or E.size != sp_meta_bytes(M, K):
        raise ValueError("operand sizes do not match (M, N, K)")
    return As, E, B


def gemm_relu_sp_ref(As, E, B, M, N, K, dtype, transB=0, relu=True, rows=None, cols=None):
    """max(A·op(B), 0) in binary64 for a 2:4 sparse A given as (As, E): the
    full (M, N) product, or (values, absum) at positions (rows[t], cols[t])."""
    lib = _load()
    As, E, B = _sp_check(As, E, B, M, N, K, dtype, transB)
    if rows is None:
        out = np.empty((M, N), dtype=np.float64)
        rc = lib.oracle_gemm_sp_relu(_vptr(As), _vptr(E), _vptr(B), None, None, 0,
                                     _ptr(out, ctypes.c_double), None, M, N, K, dtype, transB,
                                     1 if relu else 0)
        if rc != 0:
            raise ValueError("oracle_gemm_sp_relu failed (%d)" % rc)
        return out
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.empty(rows.shape, dtype=np.float64)
    absum = np.empty(rows.shape, dtype=np.float64)
    rc = lib.oracle_gemm_sp_relu(_vptr(As), _vptr(E), _vptr(B), _ptr(rows, ctypes.c_int64),
                                 _ptr(cols, ctypes.c_int64), rows.size,
                                 _ptr(out, ctypes.c_double), _ptr(absum, ctypes.c_double),
                                 M, N, K, dtype, transB, 1 if relu else 0)
    if rc != 0:
        raise ValueError("oracle_gemm_sp_relu failed (%d)" % rc)
    return out, absum


def gemm_relu_sp_fraction(As, E, B, M, N, K, dtype, transB=0, relu=True):
    """Exact rational sparse product (tiny shapes): the metadata read with
    Python integer operations, the values decoded as in gemm_relu_fraction."""
    As = _bits(As, dtype).reshape(M, K // 2)
    E = np.ascontiguousarray(E, dtype=np.uint8).reshape(-1)
    Bv = _exact(_bits(B, dtype).reshape(-1), dtype)
    out = []
    for i in range(M):
        row = [Fraction(0)] * K
        vals = _exact(As[i], dtype)
        for q in range(K // 4):
            byte = int(E[(q // 16) * M * 8 + i * 8 + (q % 16) // 2])
            nib = (byte >> 4) if q % 2 else (byte & 15)
            p0, p1 = nib & 3, nib >> 2
            if p0 >= p1:
                raise ValueError("metadata nibble with p0 >= p1")
            row[4 * q + p0] = vals[2 * q]
            row[4 * q + p1] = vals[2 * q + 1]
        r = []
        for j in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += row[k] * Bv[j * K + k if transB else k * N + j]
            r.append(max(acc, Fraction(0)) if relu else acc)
        out.append(r)
    return out
