"""Pins of the CPU oracle against facts fixed outside it (no GPU).

Every check here compares the oracle with something it does not compute
itself: hand-worked fixtures, exact rational brute force, closed forms,
algebraic identities and exhaustive decoder tables from numpy.  The operation
is the fused GEMM + ReLU of page "TileLang：GPU/NPU 通用算子 DSL", §3.2 (GPU
minimal example) and §3.3 (Ascend 950 version: B stored (N,K), transpose_B).
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl
from tests.helpers import read_golden

F16, BF16 = oracle.F16, oracle.BF16


def enc(vals, dtype):
    return wl.encode(np.asarray(vals, dtype=np.float64), dtype)


# ---------------------------------------------------------------- P1 decoders
def test_decode_f16_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, F16)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signs of zero survive decoding
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_decode_bf16_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, BF16)
    want = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


# ---------------------------------------------------------- hand-worked golden
@pytest.mark.parametrize("name", ["handworked_f16_2x2x3.txt",
                                  "handworked_bf16_transB_2x3x2.txt",
                                  "handworked_f16_extremes_2x1x2.txt",
                                  "handworked_f16_zero_k.txt"])
def test_golden_handworked(name):
    g = read_golden(name)
    dtype = {"f16": F16, "bf16": BF16}[g["dtype"]]
    M, N, K = g["M"], g["N"], g["K"]
    A = enc([float(x) for r in g["A"] for x in r], dtype) if K else np.zeros(0, np.uint16)
    B = enc([float(x) for r in g["B"] for x in r], dtype) if K else np.zeros(0, np.uint16)
    # inputs must be exact in the 16-bit format, else the fixture is wrong
    assert [Fraction(float(v)) for v in oracle.decode(A, dtype)] == \
        [x for r in g["A"] for x in r]
    C = oracle.gemm_relu_ref(A, B, M, N, K, dtype, g["transB"])
    assert [[Fraction(float(v)) for v in row] for row in C] == g["C"]
    Cf = oracle.gemm_relu_fraction(A, B, M, N, K, dtype, g["transB"])
    assert Cf == g["C"]


# -------------------------------------------------------------- P2 identities
@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("transB", [0, 1])
def test_identity_right(dtype, transB):
    M, K = 5, 7
    A = wl.uniform((M, K), 11, dtype)
    I = enc(np.eye(K), dtype)            # symmetric, so (K,N) and (N,K) agree
    C = oracle.gemm_relu_ref(A, I, M, K, K, dtype, transB)
    a = oracle.decode(A, dtype)
    assert np.array_equal(C, np.maximum(a, 0.0))


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_identity_left(dtype):
    M, N = 6, 9
    B = wl.uniform((M, N), 12, dtype)    # (K,N) with K = M
    I = enc(np.eye(M), dtype)
    C = oracle.gemm_relu_ref(I, B, M, N, M, dtype, 0)
    assert np.array_equal(C, np.maximum(oracle.decode(B, dtype), 0.0))
    # with B stored (N,K), A = I gives relu of B read column-wise
    Bt = wl.uniform((N, M), 13, dtype)
    C = oracle.gemm_relu_ref(I, Bt, M, N, M, dtype, 1)
    assert np.array_equal(C, np.maximum(oracle.decode(Bt, dtype).T, 0.0))


# ------------------------------------------------------------- P3 permutation
@pytest.mark.parametrize("transB", [0, 1])
def test_permutation(transB):
    M, K = 4, 11
    rng = np.random.default_rng(5)
    pi = rng.permutation(K)
    P = np.zeros((K, K))
    P[np.arange(K), pi] = 1.0            # P[k, pi(k)] = 1: column pi(k) of C is column k of A
    A = wl.uniform((M, K), 14, F16)
    Bm = P.T if transB else P
    C = oracle.gemm_relu_ref(A, enc(Bm, F16), M, K, K, F16, transB)
    a = np.maximum(oracle.decode(A, F16), 0.0)
    for k in range(K):
        assert np.array_equal(C[:, pi[k]], a[:, k])


# ------------------------------------------------------------ P4 closed forms
@pytest.mark.parametrize("transB", [0, 1])
def test_rank_one_closed_form(transB):
    # A = u p^T, B = q v^T  =>  ref_ij = max((p.q) u_i v_j, 0)
    u = [1, -2, 0.5, 3, -0.25]
    p = [1, 2, -1, 0.5, 4, -3, 1.5]
    q = [2, -1, 1, 0.25, -0.5, 1, 2]
    v = [-1, 0.5, 2, -4, 1, 3]
    M, K, N = len(u), len(p), len(v)
    A = np.outer(u, p)
    Bkn = np.outer(q, v)
    B = Bkn.T if transB else Bkn
    C = oracle.gemm_relu_ref(enc(A, F16), enc(B, F16), M, N, K, F16, transB)
    pq = sum(Fraction(a) * Fraction(b) for a, b in zip(p, q))
    for i in range(M):
        for j in range(N):
            want = max(pq * Fraction(u[i]) * Fraction(v[j]), Fraction(0))
            assert Fraction(float(C[i, j])) == want


@pytest.mark.parametrize("K", [1, 255, 256, 4096, 8192])
def test_all_ones_gives_K(K):
    M, N = 3, 5
    A = enc(np.ones((M, K)), F16)
    B = enc(np.ones((K, N)), F16)
    C = oracle.gemm_relu_ref(A, B, M, N, K, F16, 0)
    assert np.all(C == K)
    Cn = oracle.gemm_relu_ref(enc(-np.ones((M, K)), F16), B, M, N, K, F16, 0)
    assert np.all(Cn == 0.0) and not np.any(np.signbit(Cn))


# ------------------------------------------------------------ P5 cancellation
@pytest.mark.parametrize("K", [2, 64, 1000])
def test_alternating_rows_cancel(K):
    M, N = 4, 6
    sign = np.where(np.arange(K) % 2 == 0, 1.0, -1.0)
    a = np.outer([1.0, 0.5, 2.0, -3.0], sign)          # A_ik = a_i (-1)^k
    b = np.outer(np.ones(K), [1.0, -2.0, 0.25, 4.0, 1.5, -1.0])   # B_kj = b_j
    C = oracle.gemm_relu_ref(enc(a, F16), enc(b, F16), M, N, K, F16, 0)
    assert np.all(C == 0.0)


# -------------------------------------------------------------- P6 ReLU alone
@pytest.mark.parametrize("transB", [0, 1])
def test_relu_identities(transB):
    M, N, K = 13, 17, 29
    A, B = wl.make_inputs(M, N, K, F16, transB, "uniform", 77)
    negA = A ^ np.uint16(0x8000)                        # -A by the sign bit
    X = oracle.gemm_relu_ref(A, B, M, N, K, F16, transB, relu=False)
    Rp = oracle.gemm_relu_ref(A, B, M, N, K, F16, transB)
    Rn = oracle.gemm_relu_ref(negA, B, M, N, K, F16, transB)
    assert np.array_equal(Rp - Rn, X)
    assert np.array_equal(Rp + Rn, np.abs(X))
    assert np.all(Rp >= 0) and np.all(Rn >= 0)
    assert np.any(X < 0) and np.any(X > 0)


# ----------------------------------------------------- P7 exact brute force
def test_bruteforce_all_small_shapes():
    rng = np.random.default_rng(2024)
    grid = np.arange(-8, 9) / 4.0                      # exact in both formats
    for M, N, K in itertools.product(range(1, 7), repeat=3):
        for dtype, transB in ((F16, 0), (BF16, 1)):
            A = enc(rng.choice(grid, size=M * K), dtype)
            B = enc(rng.choice(grid, size=K * N), dtype)
            C = oracle.gemm_relu_ref(A, B, M, N, K, dtype, transB)
            want = oracle.gemm_relu_fraction(A, B, M, N, K, dtype, transB)
            got = [[Fraction(float(x)) for x in row] for row in C]
            assert got == want, (M, N, K, dtype, transB)


@pytest.mark.parametrize("transB", [0, 1])
def test_bruteforce_exhaustive_2x2x2(transB):
    # all 3^8 assignments of {-1, 0, 1} to the 4 + 4 operand entries
    vals = np.array([-1.0, 0.0, 1.0])
    for combo in itertools.product(range(3), repeat=8):
        a = vals[list(combo[:4])]
        b = vals[list(combo[4:])]
        A, B = enc(a, F16), enc(b, F16)
        C = oracle.gemm_relu_ref(A, B, 2, 2, 2, F16, transB)
        am = a.reshape(2, 2)
        bm = b.reshape(2, 2)
        bkn = bm.T if transB else bm
        for i in range(2):
            for j in range(2):
                s = int(am[i, 0] * bkn[0, j] + am[i, 1] * bkn[1, j])
                assert C[i, j] == max(s, 0)


# ---------------------------------------------------- P8 transB equivalence
@pytest.mark.parametrize("dtype", [F16, BF16])
def test_transB_equivalence(dtype):
    M, N, K = 19, 23, 37
    A = wl.uniform((M, K), 31, dtype)
    B = wl.uniform((K, N), 32, dtype)
    Bt = np.ascontiguousarray(B.T)
    C0 = oracle.gemm_relu_ref(A, B, M, N, K, dtype, 0)
    C1 = oracle.gemm_relu_ref(A, Bt, M, N, K, dtype, 1)
    assert np.array_equal(C0.view(np.uint64), C1.view(np.uint64))


# ------------------------------------------------------- P9 power-of-two scale
@pytest.mark.parametrize("s", [-3, 1, 4])
def test_power_of_two_scaling(s):
    M, N, K = 9, 10, 21
    A = wl.uniform((M, K), 41, F16, lo=-1.0, hi=1.0)
    B = wl.uniform((K, N), 42, F16)
    a = A.view(np.float16).astype(np.float64)
    As = enc(a * 2.0 ** s, F16)
    # only exact scalings are meaningful: no element may under- or overflow
    a_back = As.view(np.float16).astype(np.float64) / 2.0 ** s
    keep = a_back == a
    A2 = np.where(keep, A, np.uint16(0))
    As2 = np.where(keep, As, np.uint16(0))
    C = oracle.gemm_relu_ref(A2, B, M, N, K, F16, 0)
    Cs = oracle.gemm_relu_ref(As2, B, M, N, K, F16, 0)
    assert np.array_equal(Cs, C * 2.0 ** s)


# ---------------------------------------------- sampled entry and error sums
def test_sampled_matches_full_and_absum():
    M, N, K = 37, 41, 53
    for transB, dtype in ((0, F16), (1, BF16)):
        A, B = wl.make_inputs(M, N, K, dtype, transB, "uniform", 9)
        C = oracle.gemm_relu_ref(A, B, M, N, K, dtype, transB)
        rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        v, absum = oracle.gemm_relu_ref_at(A, B, rows.ravel(), cols.ravel(), M, N, K,
                                           dtype, transB)
        assert np.array_equal(v.reshape(M, N), C)
        a = np.abs(oracle.decode(A, dtype).reshape(M, K))
        b = np.abs(oracle.decode(B, dtype).reshape((N, K) if transB else (K, N)))
        S = a @ (b.T if transB else b)
        assert np.allclose(absum.reshape(M, N), S, rtol=1e-12, atol=0)


def test_absum_matmul_form_matches_the_dot_products():
    """The full-size absum (library matmul of decoded magnitudes) against the
    per-position absum of the dot-product loop, and against the bound's
    defining property S >= |sum|."""
    M, N, K = 29, 33, 301
    for transB, dtype in ((0, F16), (1, BF16), (1, F16)):
        A, B = wl.make_inputs(M, N, K, dtype, transB, "uniform", 11)
        S = oracle.gemm_absum_matmul(A, B, M, N, K, dtype, transB)
        rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        _, absum = oracle.gemm_relu_ref_at(A, B, rows.ravel(), cols.ravel(), M, N, K,
                                           dtype, transB)
        assert S.shape == (M, N)
        assert np.allclose(S, absum.reshape(M, N), rtol=1e-12, atol=0)
        X = oracle.gemm_relu_ref(A, B, M, N, K, dtype, transB, relu=False)
        assert np.all(S >= np.abs(X))


def test_integer_inputs_are_exact_against_fractions():
    M, N, K = 7, 5, 300
    A, B = wl.make_inputs(M, N, K, F16, 0, "uniform", 3, int_values=True)
    C = oracle.gemm_relu_ref(A, B, M, N, K, F16, 0)
    want = oracle.gemm_relu_fraction(A, B, M, N, K, F16, 0)
    assert [[Fraction(float(x)) for x in r] for r in C] == want


def test_rejects_bad_arguments():
    A = np.zeros(4, np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm_relu_ref(A, A, 2, 2, 2, 7, 0)       # bad dtype
    with pytest.raises(ValueError):
        oracle.gemm_relu_ref(A, A, 2, 2, 2, F16, 2)     # bad transB
    with pytest.raises(ValueError):
        oracle.gemm_relu_ref_at(A, A, [2], [0], 2, 2, 2, F16)   # row out of range


def test_empty_shapes():
    z = np.zeros(0, np.uint16)
    assert oracle.gemm_relu_ref(z, z, 0, 5, 0, F16).shape == (0, 5)
    C = oracle.gemm_relu_ref(z, z, 3, 4, 0, F16)
    assert np.all(C == 0) and not np.any(np.signbit(C))


# --------------------------------------- the library-matmul form of the oracle
@pytest.mark.parametrize("transB,dtype", [(0, F16), (1, BF16), (1, F16), (0, BF16)])
def test_matmul_form_matches_loop_exactly_on_integers(transB, dtype):
    M, N, K = 45, 38, 517
    A, B = wl.make_inputs(M, N, K, dtype, transB, "uniform", 21, int_values=True)
    C1 = oracle.gemm_relu_ref(A, B, M, N, K, dtype, transB)
    C2 = oracle.gemm_relu_ref_matmul(A, B, M, N, K, dtype, transB)
    assert np.array_equal(C1, C2) and not np.any(np.signbit(C2))


def test_matmul_form_close_to_loop_on_floats():
    M, N, K = 33, 29, 1000
    A, B = wl.make_inputs(M, N, K, F16, 0, "uniform", 22)
    C1 = oracle.gemm_relu_ref(A, B, M, N, K, F16, 0)
    C2 = oracle.gemm_relu_ref_matmul(A, B, M, N, K, F16, 0)
    # two binary64 summation orders of K products: relative gap ~ K * 2^-53
    assert np.allclose(C1, C2, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ 8-bit inputs
F8E4M3, F8E5M2 = oracle.F8E4M3, oracle.F8E5M2


@pytest.mark.parametrize("dtype", [F8E4M3, F8E5M2])
def test_decode_fp8_exhaustive_against_torch(dtype):
    """All 256 patterns against torch's CPU float8 types (a library decoder)."""
    import torch
    bits = np.arange(256, dtype=np.uint8)
    got = oracle.decode(bits, dtype)
    fmt = torch.float8_e4m3fn if dtype == F8E4M3 else torch.float8_e5m2
    want = torch.from_numpy(bits.copy()).view(fmt).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.signbit(got[0x80]) and not np.signbit(got[0])


def test_decode_e5m2_is_the_top_byte_of_binary16():
    """E5M2 has binary16's sign and exponent fields and its 2 leading fraction
    bits: pattern c means the binary16 pattern c << 8."""
    bits = np.arange(256, dtype=np.uint8)
    got = oracle.decode(bits, F8E5M2)
    want = oracle.decode(bits.astype(np.uint16) << 8, F16)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_decode_e4m3_landmarks():
    bits = np.arange(256, dtype=np.uint8)
    v = oracle.decode(bits, F8E4M3)
    assert v[0x38] == 1.0 and v[0xB8] == -1.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0          # largest finite
    assert v[0x08] == 2.0 ** -6                              # smallest normal
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9  # subnormals
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(v).sum() == 254                       # no infinities
    assert np.all(np.diff(v[:0x7F]) > 0)                     # monotone over the positives


@pytest.mark.parametrize("dtype", [F8E4M3, F8E5M2])
@pytest.mark.parametrize("transB", [0, 1])
def test_bruteforce_fp8_small_shapes(dtype, transB):
    """Exact rational brute force (decoded through torch) on random 8-bit
    patterns, every shape up to 4 x 4 x 5.  Values are kept to zero and
    2^-8 <= |x| <= 2^8 so that every partial sum is exact in binary64 (E5M2's
    full range would span more than 53 bits of products)."""
    rng = np.random.default_rng(77 + dtype)
    vals = oracle.decode(np.arange(256, dtype=np.uint8), dtype)
    with np.errstate(invalid="ignore"):
        ok = (vals == 0) | ((np.abs(vals) >= 2.0 ** -8) & (np.abs(vals) <= 2.0 ** 8))
    finite = np.flatnonzero(ok)
    for M, N, K in itertools.product(range(1, 5), range(1, 5), range(0, 6)):
        A = rng.choice(finite, size=M * K).astype(np.uint8)
        B = rng.choice(finite, size=K * N).astype(np.uint8)
        got = oracle.gemm_relu_ref(A, B, M, N, K, dtype, transB)
        want = oracle.gemm_relu_fraction(A, B, M, N, K, dtype, transB)
        assert [[Fraction(float(x)) for x in row] for row in got] == want


@pytest.mark.parametrize("dtype", [F8E4M3, F8E5M2])
def test_fp8_transB_and_matmul_form(dtype):
    M, N, K = 9, 11, 70
    A = wl.integers((M, K), 5, dtype)
    Bkn = wl.integers((K, N), 6, dtype)
    Bnk = np.ascontiguousarray(Bkn.reshape(K, N).T)
    ref = oracle.gemm_relu_ref(A, Bkn, M, N, K, dtype, 0)
    assert np.array_equal(ref, oracle.gemm_relu_ref(A, Bnk, M, N, K, dtype, 1))
    assert np.array_equal(ref, oracle.gemm_relu_ref_matmul(A, Bkn, M, N, K, dtype, 0))
    a = wl.integers((M, K), 5, F16)
    b = wl.integers((K, N), 6, F16)
    # the same integers through the binary16 path
    assert np.array_equal(ref, oracle.gemm_relu_ref(a, b, M, N, K, F16, 0))


def test_fp8_inputs_must_be_bytes():
    with pytest.raises(TypeError):
        oracle.gemm_relu_ref(np.zeros(4, np.uint16), np.zeros(4, np.uint16), 2, 2, 2, F8E4M3)


# ------------------------------------------------ block-scaled (MX) inputs
MX_E4M3, MX_E5M2, MX_E2M1 = oracle.MX_E4M3, oracle.MX_E5M2, oracle.MX_E2M1
# the OCP E2M1 value table, codes 0..7 (sign in bit 3)
E2M1_SPEC = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_decode_e2m1_against_the_spec_table():
    for code in range(16):
        v = E2M1_SPEC[code & 7]
        got = oracle.dec_e2m1(code)
        assert got == (-v if code & 8 else v)
        assert np.signbit(got) == bool(code & 8)


def test_decode_e8m0():
    import math
    for e in range(255):
        assert oracle.dec_e8m0(e) == math.ldexp(1.0, e - 127)
    assert math.isnan(oracle.dec_e8m0(255))


def _random_mx(M, N, K, fmt, rng, scale_spread=6):
    rb = K // 2 if fmt == MX_E2M1 else K
    if fmt == MX_E2M1:
        A = rng.integers(0, 256, size=(M, rb)).astype(np.uint8)
        B = rng.integers(0, 256, size=(N, rb)).astype(np.uint8)
    else:
        vals = oracle.decode(np.arange(256, dtype=np.uint8), F8E4M3 if fmt == MX_E4M3 else F8E5M2)
        with np.errstate(invalid="ignore"):
            ok = np.flatnonzero((vals == 0) | ((np.abs(vals) >= 2.0 ** -6) & (np.abs(vals) <= 64)))
        A = rng.choice(ok, size=(M, rb)).astype(np.uint8)
        B = rng.choice(ok, size=(N, rb)).astype(np.uint8)
    SA = rng.integers(127 - scale_spread, 128 + scale_spread, size=(M, K // 32)).astype(np.uint8)
    SB = rng.integers(127 - scale_spread, 128 + scale_spread, size=(N, K // 32)).astype(np.uint8)
    return A, SA, B, SB


@pytest.mark.parametrize("fmt", [MX_E4M3, MX_E5M2, MX_E2M1])
def test_mx_bruteforce_small_shapes(fmt):
    """Exact rational brute force with per-block scales (its own E2M1 table,
    torch's float8 types, Fraction powers of two)."""
    rng = np.random.default_rng(31 + fmt)
    for M, N, K in [(1, 1, 32), (2, 3, 64), (3, 2, 96), (4, 4, 32)]:
        A, SA, B, SB = _random_mx(M, N, K, fmt, rng)
        got = oracle.gemm_relu_mx_ref(A, SA, B, SB, M, N, K, fmt)
        want = oracle.gemm_relu_mx_fraction(A, SA, B, SB, M, N, K, fmt)
        assert [[Fraction(float(x)) for x in row] for row in got] == want


@pytest.mark.parametrize("fmt,plain", [(MX_E4M3, F8E4M3), (MX_E5M2, F8E5M2)])
def test_mx8_with_unit_scales_is_the_plain_fp8_product(fmt, plain):
    rng = np.random.default_rng(41)
    M, N, K = 7, 9, 96
    A, _, B, _ = _random_mx(M, N, K, fmt, rng)
    one_a = np.full((M, K // 32), 127, np.uint8)
    one_b = np.full((N, K // 32), 127, np.uint8)
    got = oracle.gemm_relu_mx_ref(A, one_a, B, one_b, M, N, K, fmt)
    assert np.array_equal(got, oracle.gemm_relu_ref(A, B, M, N, K, plain, 1))


def test_mxfp4_with_unit_scales_is_the_plain_product_of_its_values():
    """E2M1 values are exact in binary16: the same product through the
    16-bit definition, with the nibbles unpacked by hand (even k low)."""
    rng = np.random.default_rng(43)
    M, N, K = 5, 6, 64
    A, _, B, _ = _random_mx(M, N, K, MX_E2M1, rng)

    def unpack(x):
        nib = np.stack([x & 0xF, x >> 4], axis=-1).reshape(x.shape[0], -1)
        mag = np.array(E2M1_SPEC)[nib & 7]
        return np.where(nib & 8, -mag, mag)

    a16 = enc(unpack(A), F16)
    b16 = enc(unpack(B), F16)
    ones = (np.full((M, K // 32), 127, np.uint8), np.full((N, K // 32), 127, np.uint8))
    got = oracle.gemm_relu_mx_ref(A, ones[0], B, ones[1], M, N, K, MX_E2M1)
    assert np.array_equal(got, oracle.gemm_relu_ref(a16, b16, M, N, K, F16, 1))


@pytest.mark.parametrize("fmt", [MX_E4M3, MX_E2M1])
def test_mx_block_scale_pulls_out(fmt):
    """Raising every scale of A's row i by d multiplies row i by 2^d; raising
    the scale of one block only scales that block's partial sum."""
    rng = np.random.default_rng(47)
    M, N, K = 4, 5, 64
    A, SA, B, SB = _random_mx(M, N, K, fmt, rng, scale_spread=3)
    base = oracle.gemm_relu_mx_ref(A, SA, B, SB, M, N, K, fmt)
    SA2 = SA.copy()
    SA2[2, :] += 3
    got = oracle.gemm_relu_mx_ref(A, SA2, B, SB, M, N, K, fmt)
    assert np.array_equal(got[2], base[2] * 8.0)
    assert np.array_equal(np.delete(got, 2, axis=0), np.delete(base, 2, axis=0))
    # one block: the no-ReLU sums split into per-block parts
    full = oracle.gemm_relu_mx_ref(A, SA, B, SB, M, N, K, fmt, relu=False)
    SA3 = SA.copy()
    SA3[:, 1] += 1
    bumped = oracle.gemm_relu_mx_ref(A, SA3, B, SB, M, N, K, fmt, relu=False)
    SA0 = SA.copy()
    SA0[:, 1] = 0                                  # block 1 scaled to 2^-127: negligible
    part0 = oracle.gemm_relu_mx_ref(A, SA0, B, SB, M, N, K, fmt, relu=False)
    assert np.allclose(bumped, full + (full - part0), rtol=0, atol=1e-30)


@pytest.mark.parametrize("fmt", [MX_E4M3, MX_E5M2, MX_E2M1])
def test_mx_sampled_matches_full_and_absum(fmt):
    """The block-scaled oracle's position mode (the one full-size GPU checks
    call) against its full mode, value for value at every position and at a
    shuffled list with repeats; its absum against sum_k |xa a xb b| built here
    from torch's float8 decoding (E4M3 / E5M2) or the OCP table (E2M1) and
    2^(e - 127) scales, by numpy's binary64 matmul.  A NaN scale (e = 255)
    makes its row's unclamped sums and absum NaN in both modes and nothing
    else."""
    import torch
    rng = np.random.default_rng(53 + fmt)
    M, N, K = 13, 11, 128
    A, SA, B, SB = _random_mx(M, N, K, fmt, rng, scale_spread=5)
    SA[4, 2] = 255
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    rows, cols = rows.ravel(), cols.ravel()
    perm = rng.permutation(np.concatenate([np.arange(M * N), rng.integers(0, M * N, 40)]))
    for relu in (True, False):
        full = oracle.gemm_relu_mx_ref(A, SA, B, SB, M, N, K, fmt, relu=relu)
        v, absum = oracle.gemm_relu_mx_ref(A, SA, B, SB, M, N, K, fmt, relu=relu, rows=rows, cols=cols)
        assert np.array_equal(v.reshape(M, N), full, equal_nan=True)
        v2, absum2 = oracle.gemm_relu_mx_ref(A, SA, B, SB, M, N, K, fmt, relu=relu,
                                             rows=rows[perm], cols=cols[perm])
        assert np.array_equal(v2, full.reshape(-1)[perm], equal_nan=True)
        assert np.array_equal(absum2, absum[perm], equal_nan=True)
    assert np.all(np.isnan(full[4])) and not np.any(np.isnan(np.delete(full, 4, axis=0)))

    def values(x):
        if fmt == MX_E2M1:
            nib = np.stack([x & 0xF, x >> 4], axis=-1).reshape(x.shape[0], -1)
            mag = np.array(E2M1_SPEC)[nib & 7]
            return np.where(nib & 8, -mag, mag)
        t = torch.from_numpy(np.ascontiguousarray(x))
        f8 = torch.float8_e4m3fn if fmt == MX_E4M3 else torch.float8_e5m2
        return t.view(f8).to(torch.float64).numpy()

    def scaled(x, sx):
        with np.errstate(invalid="ignore"):
            scale = np.where(sx == 255, np.nan, np.ldexp(1.0, sx.astype(np.int64) - 127))
        return values(x) * np.repeat(scale, 32, axis=1)

    S = np.abs(scaled(A, SA)) @ np.abs(scaled(B, SB)).T
    assert np.isnan(absum.reshape(M, N)[4]).all()
    keep = np.arange(M) != 4
    assert np.allclose(absum.reshape(M, N)[keep], S[keep], rtol=1e-12, atol=0)
    assert np.all(absum.reshape(M, N)[keep] >= np.abs(full[keep]))


def test_mx_rejects_partial_blocks():
    with pytest.raises(ValueError):
        oracle.gemm_relu_mx_ref(np.zeros(40, np.uint8), np.zeros(2, np.uint8),
                                np.zeros(40, np.uint8), np.zeros(2, np.uint8), 1, 1, 40, MX_E4M3)


# ------------------------------------------------------- 2:4 sparse A (NEXT)
# The sparse product of the T.gemm_sp item (page "TileLang：GPU/NPU 通用算子
# DSL", §4.1 timeline; page "从 TVM 到 TileLang…", §四: A compressed with its
# metadata E): (As, E) decode to a plain A, then the same definition.
def test_sp_golden_handworked():
    g = read_golden("handworked_sp_f16_2x2x8.txt")
    M, N, K = g["M"], g["N"], g["K"]
    As = enc([float(x) for r in g["AS"] for x in r], F16)
    E = np.array([int(x) for r in g["E"] for x in r], dtype=np.uint8)
    B = enc([float(x) for r in g["B"] for x in r], F16)
    C = oracle.gemm_relu_sp_ref(As, E, B, M, N, K, F16, g["transB"])
    assert [[Fraction(float(v)) for v in row] for row in C] == g["C"]
    assert oracle.gemm_relu_sp_fraction(As, E, B, M, N, K, F16, g["transB"]) == g["C"]


def test_sp_metadata_blocks_by_hand():
    """E blocked by 64 columns of K, built byte by byte: row 1's group 17 (block
    1, byte 0, high nibble) keeps positions 2, 3; everything else keeps 0, 1."""
    M, N, K = 2, 1, 128
    E = np.full(2 * M * 8, 0x44, dtype=np.uint8)       # nibble 4 = positions 0, 1
    E[1 * M * 8 + 1 * 8 + 0] = 0x4 | (0xE << 4)         # row 1, group 17 -> (2, 3)
    As = enc(np.ones(M * K // 2), F16)
    b = np.zeros(K)
    b[4 * 17 + 2] = 1.0
    b[4 * 17 + 3] = 10.0
    B = enc(b, F16)
    C = oracle.gemm_relu_sp_ref(As, E, B, M, N, K, F16, 0)
    assert C.tolist() == [[0.0], [11.0]]
    # the same byte in block 0 is row 1's groups 0 and 1
    E2 = np.full(2 * M * 8, 0x44, dtype=np.uint8)
    E2[1 * 8 + 0] = 0x4 | (0xE << 4)
    b2 = np.zeros(K)
    b2[4 + 2] = 1.0
    B2 = enc(b2, F16)
    assert oracle.gemm_relu_sp_ref(As, E2, B2, M, N, K, F16, 0).tolist() == [[0.0], [1.0]]


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("transB", [0, 1])
@pytest.mark.parametrize("M,N,K", [(3, 5, 4), (7, 6, 64), (5, 9, 68), (4, 3, 200)])
def test_sp_equals_dense_product_of_its_decompression(dtype, transB, M, N, K):
    """A random 2:4 matrix given compressed equals the dense oracle on the plain
    matrix it encodes (integer values: both sums exact)."""
    rng = np.random.default_rng(1000 + M * N + K)
    vals, positions, dense = wl.sp_random(M, K, rng, int_values=True)
    b = rng.integers(-3, 4, size=wl.b_shape(M, N, K, transB)).astype(np.float64)
    As, E, B = enc(vals, dtype), wl.sp_pack(positions, M, K), enc(b, dtype)
    got = oracle.gemm_relu_sp_ref(As, E, B, M, N, K, dtype, transB)
    want = oracle.gemm_relu_ref(enc(dense, dtype), B, M, N, K, dtype, transB)
    assert np.array_equal(got, want)
    # at chosen positions too, with the absolute-value sum
    rows, cols = np.array([0, M - 1]), np.array([N - 1, 0])
    at, absum = oracle.gemm_relu_sp_ref(As, E, B, M, N, K, dtype, transB, rows=rows, cols=cols)
    assert np.array_equal(at, want[rows, cols])
    bmat = b if not transB else b.T
    assert np.array_equal(absum, np.abs(dense[rows] * bmat[:, cols].T).sum(axis=1))


@pytest.mark.parametrize("M,N,K", [(1, 1, 4), (2, 3, 8), (3, 2, 68)])
@pytest.mark.parametrize("transB", [0, 1])
def test_sp_fraction_bruteforce(M, N, K, transB):
    rng = np.random.default_rng(2000 + M + N + K)
    vals, positions, _ = wl.sp_random(M, K, rng)
    b = rng.uniform(-1, 1, size=wl.b_shape(M, N, K, transB))
    As, E, B = enc(vals, F16), wl.sp_pack(positions, M, K), enc(b, F16)
    got = oracle.gemm_relu_sp_ref(As, E, B, M, N, K, F16, transB)
    exact = oracle.gemm_relu_sp_fraction(As, E, B, M, N, K, F16, transB)
    # each product of two fp16 values is exact in binary64; K / 2 terms
    for i in range(M):
        for j in range(N):
            assert abs(Fraction(float(got[i][j])) - exact[i][j]) <= Fraction(K, 2 ** 40)


def test_sp_position_sum_closed_form():
    """All stored values 1 and b(k, 0) = k: C[i][0] = sum_q (8 q + p0 + p1)."""
    M, K = 6, 136
    rng = np.random.default_rng(31)
    _, positions, _ = wl.sp_random(M, K, rng)
    As = enc(np.ones((M, K // 2)), F16)
    B = enc(np.arange(K, dtype=np.float64).reshape(K, 1), F16)
    C = oracle.gemm_relu_sp_ref(As, wl.sp_pack(positions, M, K), B, M, 1, K, F16, 0)
    q = np.arange(K // 4)
    want = (8 * q[None, :] + positions[..., 0] + positions[..., 1]).sum(axis=1)
    assert np.array_equal(C[:, 0], want.astype(np.float64))


def test_sp_rejects_bad_metadata_and_partial_groups():
    M, N, K = 1, 1, 8
    As, B = enc(np.ones(4), F16), enc(np.ones(8), F16)
    E = np.zeros(8, np.uint8)
    E[0] = 0x4 | (0x5 << 4)                  # group 1: p0 = 1, p1 = 1
    with pytest.raises(ValueError):
        oracle.gemm_relu_sp_ref(As, E, B, M, N, K, F16, 0)
    with pytest.raises(ValueError):
        oracle.gemm_relu_sp_ref(As, np.zeros(8, np.uint8), B, M, N, 6, F16, 0)
