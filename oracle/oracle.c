/*
 * CPU oracle for the fused dense GEMM + ReLU — TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may
 * load this library.  The GPU product path never calls it and shares no code,
 * header, table or helper with it.
 *
 * What it computes (page "TileLang：GPU/NPU 通用算子 DSL", §3.2 GPU minimal
 * example and §3.3 Ascend 950 version): an output tile accumulator is cleared,
 * A·B (or A·Bᵀ when B is stored (N,K) and the gemm is told transpose_B) is
 * accumulated over the whole K range, and every accumulator element is then
 * replaced by max(x, 0) before it is written out.  The tiling, the pipelined
 * K-loop and the layouts on those pages only reorder that sum, so this file
 * writes the plain definition:
 *
 *     ref[i][j] = max( sum_{k<K} a(i,k) * b(k,j), 0 )
 *
 * in IEEE binary64, with a(i,k) = dec(A[i*K+k]) and b(k,j) = dec(B[k*N+j]),
 * or dec(B[j*K+k]) when transB = 1.  The result stays binary64: no rounding to
 * the storage type of C happens here.
 *
 * dec() turns a storage pattern into its exact value.  binary16 and bfloat16
 * (16-bit patterns) and the two OCP 8-bit floating-point formats E4M3 and E5M2
 * (8-bit patterns; the "FP8 GEMM" that page's §4.1 lists among the kernels the
 * DSL covers) are decoded from their field definitions (sign, biased exponent,
 * fraction), not by reinterpreting bits through a hardware type.  The pages
 * give FP8 no scale factors, so an FP8 product here is the same definition
 * over the exact values of the 8-bit inputs.
 *
 * Block-scaled (MX) inputs — the "MXFP8 block-scaled GEMM" and "CDNA4 MXFP4"
 * of that page's §4.1 capability timeline — follow the OCP Microscaling
 * definition: every 32 consecutive elements of a row along K share one E8M0
 * scale X = 2^(e - 127), and an element's value is X times its own value.
 * Here A is (M, K), B is stored (N, K), and their scales are (M, K/32) and
 * (N, K/32) row-major byte arrays, so
 *
 *     ref[i][j] = max( sum_b XA[i][b] XB[j][b] sum_{k in block b} a(i,k) b(j,k), 0 )
 *
 * with 4-bit E2M1 elements packed two to a byte, element k of a row in the
 * low nibble of byte k/2 when k is even and in the high nibble when odd.
 *
 * 2:4 structured-sparse A — the "2:4 structured-sparse tensor core (T.gemm_sp)"
 * of that page's §4.1 timeline, whose A arrives compressed together with its
 * metadata E (page "从 TVM 到 TileLang…", §四) — is decoded back to the plain
 * matrix first, then the same definition applies.  The pages fix no format;
 * the one read here: every row of A is cut along K into groups of 4, each
 * holding its (at most) two non-zeros; As (M, K/2) keeps them, As[i][2q] and
 * As[i][2q+1] for group q, and E gives their positions p0 < p1 inside the
 * group as the nibble p0 | p1 << 2.  E is blocked by 64 columns of K: block
 * kb = q / 16 holds 8 bytes per row (M x 8 bytes), and group q of row i is
 * nibble q % 2 (low nibble first) of byte (q % 16) / 2 of row i's 8 bytes.
 * So a(i, 4q + p0) = As[i][2q], a(i, 4q + p1) = As[i][2q+1], and the other
 * two elements of the group are zero.
 *
 * Readings where the pages are silent (listed with the others in the design
 * notes): a negative sum maps to +0.0; K = 0 gives an empty sum, so every
 * output is +0.0; M = 0 or N = 0 is a no-op.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1, ORACLE_FP8_E4M3 = 3, ORACLE_FP8_E5M2 = 4 };
/* element formats of the block-scaled product */
enum { ORACLE_MX_E4M3 = 5, ORACLE_MX_E5M2 = 6, ORACLE_MX_E2M1 = 7 };

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_dec_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);              /* subnormal: f * 2^-10 * 2^-14 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);  /* (1 + f/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_dec_bf16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int f = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);             /* subnormal: f * 2^-7 * 2^-126 */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);  /* (1 + f/2^7) * 2^(e-127) */
    return sign ? -v : v;
}

/* OCP 8-bit E4M3 ("FN": finite only): 1 sign bit, 4 exponent bits (bias 7),
 * 3 fraction bits.  Exponent field 15 with fraction 7 is NaN; every other
 * pattern is finite (largest 1.75 * 2^8 = 448).  No infinities. */
double oracle_dec_e4m3(uint8_t h)
{
    int sign = (h >> 7) & 1;
    int e = (h >> 3) & 0xf;
    int f = h & 0x7;
    double v;
    if (e == 0)
        v = ldexp((double)f, -9);               /* subnormal: f * 2^-3 * 2^-6 */
    else if (e == 15 && f == 7)
        v = NAN;
    else
        v = ldexp((double)(8 + f), e - 10);     /* (1 + f/2^3) * 2^(e-7) */
    return sign ? -v : v;
}

/* OCP 8-bit E5M2: 1 sign bit, 5 exponent bits (bias 15), 2 fraction bits,
 * with IEEE infinities and NaNs at exponent field 31. */
double oracle_dec_e5m2(uint8_t h)
{
    int sign = (h >> 7) & 1;
    int e = (h >> 2) & 0x1f;
    int f = h & 0x3;
    double v;
    if (e == 0)
        v = ldexp((double)f, -16);              /* subnormal: f * 2^-2 * 2^-14 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(4 + f), e - 17);     /* (1 + f/2^2) * 2^(e-15) */
    return sign ? -v : v;
}

/* Exact value of element idx of a storage array of the given type. */
/* OCP 4-bit E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 fraction bit; all
 * 16 patterns finite (largest 1.5 * 2^2 = 6). */
double oracle_dec_e2m1(uint8_t h)
{
    int sign = (h >> 3) & 1;
    int e = (h >> 1) & 0x3;
    int f = h & 0x1;
    double v = e == 0 ? ldexp((double)f, -1)            /* subnormal: f * 2^-1 * 2^0 */
                      : ldexp((double)(2 + f), e - 2);  /* (1 + f/2) * 2^(e-1) */
    return sign ? -v : v;
}

/* OCP E8M0 scale: 2^(e - 127); e = 255 is NaN. */
double oracle_dec_e8m0(uint8_t e)
{
    return e == 255 ? NAN : ldexp(1.0, (int)e - 127);
}

static double dec_at(const void* x, int64_t idx, int dtype)
{
    switch (dtype) {
    case ORACLE_F16: return oracle_dec_f16(((const uint16_t*)x)[idx]);
    case ORACLE_BF16: return oracle_dec_bf16(((const uint16_t*)x)[idx]);
    case ORACLE_FP8_E4M3: return oracle_dec_e4m3(((const uint8_t*)x)[idx]);
    default: return oracle_dec_e5m2(((const uint8_t*)x)[idx]);
    }
}

void oracle_decode(const void* x, double* out, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = dec_at(x, i, dtype);
}

static int bad_args(const void* A, const void* B, const void* C,
                    int64_t M, int64_t N, int64_t K, int dtype, int transB)
{
    if (M < 0 || N < 0 || K < 0) return 1;
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16 && dtype != ORACLE_FP8_E4M3 &&
        dtype != ORACLE_FP8_E5M2)
        return 1;
    if (transB != 0 && transB != 1) return 1;
    if ((M > 0 && K > 0 && !A) || (N > 0 && K > 0 && !B) || (M > 0 && N > 0 && !C)) return 1;
    return 0;
}

/* b(k, j) as the definition indexes it. */
static int64_t b_index(int64_t k, int64_t j, int64_t N, int64_t K, int transB)
{
    return transB ? j * K + k : k * N + j;
}

/*
 * Full product.  C is (M, N) row-major binary64.  relu = 0 skips the max (a test
 * mode used to pin the ReLU on its own).  threads = 0 lets OpenMP choose.
 * Returns 0, or -1 on bad arguments.  *threads_used (if not NULL) receives the
 * number of threads the row loop ran on.
 */
int oracle_gemm_relu_f64(const void* A, const void* B, double* C,
                         int64_t M, int64_t N, int64_t K,
                         int dtype, int transB, int relu, int threads,
                         int* threads_used)
{
    if (bad_args(A, B, C, M, N, K, dtype, transB)) return -1;
    if (threads_used) *threads_used = 1;
    if (M == 0 || N == 0) return 0;

    /* Decode both operands once: a(i,k) and b(k,j) are exact in binary64. */
    double* Ad = (double*)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    double* Bd = (double*)malloc(sizeof(double) * (size_t)(K * N > 0 ? K * N : 1));
    if (!Ad || !Bd) { free(Ad); free(Bd); return -2; }
    oracle_decode(A, Ad, M * K, dtype);
    oracle_decode(B, Bd, K * N, dtype);

#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#endif
    int used = 1;
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        double* acc = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < M; ++i) {
            for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
            if (!transB) {
                /* i-k-j: add a(i,k) * row k of B into the row accumulator. */
                for (int64_t k = 0; k < K; ++k) {
                    double a = Ad[i * K + k];
                    const double* brow = Bd + k * N;
                    for (int64_t j = 0; j < N; ++j) acc[j] += a * brow[j];
                }
            } else {
                /* i-j: dot product of row i of A with row j of the (N,K) B. */
                for (int64_t j = 0; j < N; ++j) {
                    double s = 0.0;
                    for (int64_t k = 0; k < K; ++k) s += Ad[i * K + k] * Bd[j * K + k];
                    acc[j] = s;
                }
            }
            for (int64_t j = 0; j < N; ++j) {
                double x = acc[j];
                C[i * N + j] = relu ? (x > 0.0 ? x : 0.0) : x;
            }
        }
        free(acc);
    }
    if (threads_used) *threads_used = used;
    free(Ad);
    free(Bd);
    return 0;
}

/*
 * The same definition at n chosen output positions (rows[t], cols[t]), one dot
 * product each, for full-size problems where the whole product is too slow.
 * If absum is not NULL it also receives S = sum_k |a(i,k) * b(k,j)|, the scale
 * of the floating-point summation error bound.
 */
int oracle_gemm_relu_f64_at(const void* A, const void* B,
                            const int64_t* rows, const int64_t* cols, int64_t n,
                            double* out, double* absum,
                            int64_t M, int64_t N, int64_t K,
                            int dtype, int transB, int relu)
{
    if (bad_args(A, B, out, M, N, K, dtype, transB) || n < 0 || (n > 0 && (!rows || !cols)))
        return -1;
    for (int64_t t = 0; t < n; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < n; ++t) {
        int64_t i = rows[t], j = cols[t];
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = dec_at(A, i * K + k, dtype) * dec_at(B, b_index(k, j, N, K, transB), dtype);
            s += p;
            sa += fabs(p);
        }
        out[t] = relu ? (s > 0.0 ? s : 0.0) : s;
        if (absum) absum[t] = sa;
    }
    return 0;
}

/* Element k of a row of an MX operand (row stride in elements = K). */
static double mx_elem(const uint8_t* row, int64_t k, int fmt)
{
    if (fmt == ORACLE_MX_E2M1) {
        uint8_t byte = row[k / 2];
        return oracle_dec_e2m1((k % 2) ? (byte >> 4) : (byte & 0xf));
    }
    return fmt == ORACLE_MX_E4M3 ? oracle_dec_e4m3(row[k]) : oracle_dec_e5m2(row[k]);
}

/*
 * Block-scaled product at n positions (rows[t], cols[t]), or the full (M, N)
 * product when rows == NULL (then n is ignored and out is M x N row-major).
 * A: M x K elements, B: N x K elements (both rows along K), SA: M x K/32 and
 * SB: N x K/32 E8M0 bytes.  K must be a multiple of 32.  absum (optional)
 * receives sum_k |scaled a * scaled b|.  Returns 0 or -1 on bad arguments.
 */
int oracle_gemm_relu_mx(const void* A, const void* SA, const void* B, const void* SB,
                        const int64_t* rows, const int64_t* cols, int64_t n,
                        double* out, double* absum, int64_t M, int64_t N, int64_t K,
                        int fmt, int relu)
{
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return -1;
    if (fmt != ORACLE_MX_E4M3 && fmt != ORACLE_MX_E5M2 && fmt != ORACLE_MX_E2M1) return -1;
    if (!out || (K > 0 && M > 0 && (!A || !SA)) || (K > 0 && N > 0 && (!B || !SB))) return -1;
    const int64_t row_bytes = fmt == ORACLE_MX_E2M1 ? K / 2 : K;
    const int64_t nb = K / 32;
    const int64_t total = rows ? n : M * N;
    if (rows)
        for (int64_t t = 0; t < n; ++t)
            if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < total; ++t) {
        const int64_t i = rows ? rows[t] : t / N, j = rows ? cols[t] : t % N;
        const uint8_t* arow = (const uint8_t*)A + i * row_bytes;
        const uint8_t* brow = (const uint8_t*)B + j * row_bytes;
        double s = 0.0, sa = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            const double xa = oracle_dec_e8m0(((const uint8_t*)SA)[i * nb + b]);
            const double xb = oracle_dec_e8m0(((const uint8_t*)SB)[j * nb + b]);
            for (int64_t k = 32 * b; k < 32 * b + 32; ++k) {
                const double p = (xa * mx_elem(arow, k, fmt)) * (xb * mx_elem(brow, k, fmt));
                s += p;
                sa += fabs(p);
            }
        }
        out[t] = relu ? (s > 0.0 ? s : 0.0) : s;
        if (absum) absum[t] = sa;
    }
    return 0;
}

/*
 * 2:4 structured-sparse product, A given as (As, E) (format in the header
 * comment), B dense (K, N) or stored (N, K) when transB = 1, at n positions
 * (rows[t], cols[t]), or the full (M, N) product when rows == NULL.  K must be
 * a multiple of 4.  Row i of A is first decoded to its K plain values, then
 * the definition's sum is taken.  Returns 0, -1 on bad arguments, -3 when a
 * metadata nibble used has p0 >= p1.
 */
int oracle_gemm_sp_relu(const void* As, const void* E, const void* B,
                        const int64_t* rows, const int64_t* cols, int64_t n,
                        double* out, double* absum, int64_t M, int64_t N, int64_t K,
                        int dtype, int transB, int relu)
{
    if (M < 0 || N < 0 || K < 0 || K % 4 != 0) return -1;
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
    if (transB != 0 && transB != 1) return -1;
    if (!out || (K > 0 && M > 0 && (!As || !E)) || (K > 0 && N > 0 && !B)) return -1;
    const int64_t total = rows ? n : M * N;
    if (rows)
        for (int64_t t = 0; t < n; ++t)
            if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return -1;
    const uint8_t* e = (const uint8_t*)E;
    int bad = 0;
#pragma omp parallel
    {
        double* a = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        int64_t cur = -1;             /* row decoded into a[] */
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < total; ++t) {
            const int64_t i = rows ? rows[t] : t / N, j = rows ? cols[t] : t % N;
            if (i != cur) {
                for (int64_t k = 0; k < K; ++k) a[k] = 0.0;
                for (int64_t q = 0; q < K / 4; ++q) {
                    const uint8_t byte = e[((q / 16) * M + i) * 8 + (q % 16) / 2];
                    const int nib = (q % 2) ? (byte >> 4) : (byte & 0xf);
                    const int p0 = nib & 3, p1 = nib >> 2;
                    if (p0 >= p1) {
#pragma omp atomic write
                        bad = 1;
                    }
                    a[4 * q + p0] = dec_at(As, i * (K / 2) + 2 * q, dtype);
                    a[4 * q + p1] = dec_at(As, i * (K / 2) + 2 * q + 1, dtype);
                }
                cur = i;
            }
            double s = 0.0, sa = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double p = a[k] * dec_at(B, b_index(k, j, N, K, transB), dtype);
                s += p;
                sa += fabs(p);
            }
            out[t] = relu ? (s > 0.0 ? s : 0.0) : s;
            if (absum) absum[t] = sa;
        }
        free(a);
    }
    return bad ? -3 : 0;
}
