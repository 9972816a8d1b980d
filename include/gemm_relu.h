/*
 * gemm_relu — fused dense GEMM + ReLU on AMD Instinct MI355X (gfx950).
 *
 * C-ABI of the library libgemm_relu.so.  Plain pointers and sizes only.
 *
 * The operation is the running example of page "TileLang：GPU/NPU 通用算子 DSL"
 * (§3.2, GPU minimal example, and §3.3, Ascend 950 version):
 *
 *     C = max(A · op(B), 0)
 *
 * with 16-bit inputs, an fp32 accumulator that starts cleared (C is
 * overwritten, never accumulated into), the max taken on the fp32 sum before
 * it is converted to the storage type of C.  op(B) = B when B is stored (K, N)
 * and op(B) = Bᵀ when B is stored (N, K) (§3.3's transpose_B).  The argument
 * order (A, B, C, M, N, K) follows the gemm(A, B, C, M, N, K) call sketched on
 * page "TileLang Skill：80行Python替代500行CUDA…" (its API example).
 */
#ifndef GEMM_RELU_H
#define GEMM_RELU_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type codes. */
#define GEMM_RELU_F16  0 /* IEEE binary16 (inputs or output) */
#define GEMM_RELU_BF16 1 /* bfloat16 (inputs or output) */
#define GEMM_RELU_F32  2 /* IEEE binary32 (output only) */
/* OCP 8-bit floating point (inputs only).  §4.1 of page "TileLang：GPU/NPU 通用
 * 算子 DSL" lists an FP8 GEMM among the kernels the DSL covers but gives it no
 * scale factors: the product is the same definition over the exact values of
 * the 8-bit inputs. */
#define GEMM_RELU_F8_E4M3 3 /* E4M3 ("FN"): bias 7, largest finite 448, no infinities */
#define GEMM_RELU_F8_E5M2 4 /* E5M2: bias 15, IEEE-style infinities and NaNs */
/* Block-scaled (OCP Microscaling) element formats, for gemm_relu_mx only. */
#define GEMM_RELU_MX_E4M3 5 /* MXFP8: E4M3 elements */
#define GEMM_RELU_MX_E5M2 6 /* MXFP8: E5M2 elements */
#define GEMM_RELU_MX_E2M1 7 /* MXFP4: E2M1 elements, two per byte (even k in the low nibble) */

/* Status codes.  The library never aborts, throws or prints. */
#define GEMM_RELU_OK            0
#define GEMM_RELU_EINVAL       -1 /* bad argument: size, pointer, code, overlap */
#define GEMM_RELU_EUNSUPPORTED -2 /* valid request the library cannot run (device, size limits) */
#define GEMM_RELU_EHIP         -3 /* a HIP runtime call or kernel launch failed */
#define GEMM_RELU_ESCRATCH     -4 /* gemm_relu_noalloc: the request needs more scratch than it holds */

/*
 * gemm_relu — C[i][j] = max( sum_k A[i][k] * opB[k][j], 0 ).
 *
 * Arguments
 *   A          device pointer, M x K row-major, element type in_dtype.
 *   B          device pointer; transB == 0: K x N row-major;
 *                              transB == 1: N x K row-major (C = max(A·Bᵀ, 0)).
 *   C          device pointer, M x N row-major, element type out_dtype.  Every
 *              element is overwritten; nothing is read from C.
 *   M, N, K    sizes, >= 0 and <= INT32_MAX.  M == 0 or N == 0: nothing to do,
 *              returns GEMM_RELU_OK without touching the device.  K == 0: every
 *              element of C becomes +0 (an empty sum).
 *   in_dtype   GEMM_RELU_F16, GEMM_RELU_BF16, GEMM_RELU_F8_E4M3 or
 *              GEMM_RELU_F8_E5M2 (A and B share it).
 *   out_dtype  GEMM_RELU_F16, GEMM_RELU_BF16 or GEMM_RELU_F32.
 *   transB     0 or 1, as above.
 *   stream     a hipStream_t, or NULL for the null stream.
 *
 * Layout: dense rows, no leading-dimension arguments.  A, B and C need the
 * alignment of their element type (1 byte for the 8-bit inputs); any shape is
 * accepted.
 *
 * Numerics: products of the inputs (exact in fp32 for every input type) are
 * summed in fp32 on the matrix units (order unspecified); the fp32 sum goes
 * through max(x, 0) — a negative or zero sum gives +0 — and is rounded to
 * nearest-even into out_dtype.
 *
 * Ownership: the caller owns A, B and C; the library keeps no pointer after the
 * call returns and allocates no device memory.  (A build made with
 * GEMM_RELU_COMPARISON_CONFIGS defined also holds the stream-K comparison
 * configuration, chosen only by name, GEMM_RELU_FORCE_CONFIG=
 * d256x256x32_s4_isk: its first call on a stream allocates and zeroes a
 * 128 MiB workspace for that stream (fp32 partial tiles and arrival counters),
 * kept until the process ends.  Calls on one stream share it in stream order;
 * a call on a stream that is being captured into a graph and has no workspace
 * yet takes whole tiles instead.  The default build has no such path.)
 *
 * Execution: asynchronous on `stream`; the call returns after the launch.  A
 * device-side fault surfaces at the caller's next synchronisation.  With the
 * environment variable GEMM_RELU_SYNC=1 the call synchronises the stream and
 * reports a failure as GEMM_RELU_EHIP.
 *
 * Errors: GEMM_RELU_EINVAL for negative or too-large sizes, a NULL pointer for
 * an operand that has elements, a misaligned pointer, an unknown dtype code or
 * combination, transB not in {0, 1}, or C overlapping A or B (checked before
 * any HIP call); GEMM_RELU_EUNSUPPORTED when the current device is not gfx950;
 * GEMM_RELU_EHIP when a HIP call fails.  On error nothing is launched.
 */
int gemm_relu(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
              int in_dtype, int out_dtype, int transB, void* stream);

/*
 * gemm_relu_ws — gemm_relu with a device workspace the caller provides, which
 * lets the library split the K range of each output tile over several
 * workgroups.  The product is that of gemm_relu (page "TileLang：GPU/NPU 通用算
 * 子 DSL", §3.2); the fp32 accumulator of an output element is then formed in
 * parts, each part a sum over a contiguous K range, and the parts are added in
 * K order in fp32 before max(x, 0) and the rounding (the ReLU is never applied
 * to a part: it does not distribute over the sum).
 *
 * Used for skinny shapes (M <= 64 with few output tiles), whose (K,N) B would
 * otherwise be read as narrow column slabs, which HBM serves slowly: each part
 * reads a contiguous run of many K rows instead.  Other shapes, or a workspace
 * smaller than gemm_relu_workspace_size, run exactly as gemm_relu.  (A library
 * built with the comparison configurations also splits the last, partial
 * round of 256x256 tiles this way when GEMM_RELU_FORCE_CONFIG names
 * d256x256x32_s4_i16w8sk: the same workspace layout, two 256 KiB partial
 * tiles per workgroup of that round.)
 *
 * Arguments as for gemm_relu, plus
 *   workspace        device pointer, 256-byte aligned, disjoint from A, B and
 *                    C; or NULL (no workspace: the call is gemm_relu).
 *   workspace_bytes  its size in bytes (0: no workspace).
 *
 * Workspace contents: the first 4096 bytes are arrival counters of the split
 * tiles.  They must be zero before the workspace's first use (hipMemset once
 * after allocating it), and every call that splits leaves them zero again;
 * the rest holds fp32 partial tiles during the call and is not read before it
 * is written.  Calls that may run concurrently (other streams, or graphs
 * replayed concurrently) need workspaces of their own; calls ordered on one
 * stream may share one.  The library keeps no pointer to it.  The call
 * allocates nothing, so it may be captured into a graph.
 *
 * Numerics as for gemm_relu; the summation order is fixed for given sizes, so
 * repeated calls give the same bits.  Errors as for gemm_relu, plus EINVAL for
 * a misaligned workspace or one that overlaps A, B or C.
 */
int gemm_relu_ws(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                 int in_dtype, int out_dtype, int transB, void* workspace,
                 uint64_t workspace_bytes, void* stream);

/*
 * gemm_relu_noalloc — gemm_relu_ws for callers that cannot allocate device
 * memory or bring a workspace (code under graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a 16 MiB device array of
 * the library, one per GPU, held until the process ends; the call allocates
 * nothing.  Same arguments, results and errors as gemm_relu, plus
 * GEMM_RELU_ESCRATCH when the K split the plan would take needs more than
 * 16 MiB (gemm_relu_workspace_size bytes; never for plans chosen without a
 * forced configuration, which need at most 8 MiB + 4 KiB).
 *
 * Every call on a GPU uses that GPU's one array, which keeps what the last call
 * left: each call that splits first zeroes its arrival words (a small kernel on
 * `stream`).  Calls that overlap on one GPU (other streams, concurrently
 * replayed graphs) race on the array and give undefined results; calls ordered
 * on one stream do not.
 */
int gemm_relu_noalloc(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                      int in_dtype, int out_dtype, int transB, void* stream);

/*
 * gemm_relu_workspace_size — bytes of workspace gemm_relu_ws would use for
 * these sizes and types (0 when it would not split K; otherwise 4096 bytes of
 * counters plus 32 KiB per 64 x 128 output tile and K part), or
 * GEMM_RELU_EINVAL (negative) for invalid sizes or codes.  Host-only.
 */
int64_t gemm_relu_workspace_size(int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype,
                                 int transB);

/* Configuration name gemm_relu_ws would launch with this workspace (as
 * gemm_relu_plan; the workspace pointer is checked, never dereferenced). */
const char* gemm_relu_ws_plan(const void* A, const void* B, const void* C, int64_t M, int64_t N,
                              int64_t K, int in_dtype, int out_dtype, int transB,
                              const void* workspace, uint64_t workspace_bytes);

/* Static message for a status code (never NULL). */
const char* gemm_relu_strerror(int status);

/*
 * gemm_relu_configs — comma-separated names of the kernel configurations this
 * build of the library holds (the names gemm_relu_plan, gemm_relu_mx_plan and
 * gemm_relu_sp_plan return, and the values GEMM_RELU_FORCE_CONFIG accepts).
 * Host-only, a static string, never NULL.
 */
const char* gemm_relu_configs(void);

/*
 * gemm_relu_plan — name of the kernel configuration gemm_relu would launch for
 * these arguments, without touching the device ("none" when there is nothing
 * to launch, NULL when gemm_relu would return GEMM_RELU_EINVAL).  Host-only;
 * the pointers are inspected for alignment and overlap, never dereferenced.
 */
const char* gemm_relu_plan(const void* A, const void* B, const void* C, int64_t M, int64_t N,
                           int64_t K, int in_dtype, int out_dtype, int transB);

/*
 * gemm_relu_mx — the block-scaled product: the "MXFP8 block-scaled GEMM" and
 * "CDNA4 MXFP4" items of the §4.1 capability timeline of page "TileLang：GPU/NPU
 * 通用算子 DSL", read as the
 * OCP Microscaling (MX) definition.  Every 32 consecutive elements of a row
 * along K share one E8M0 scale (2^(e - 127); e = 255 is NaN), and
 *
 *   C[i][j] = max( sum_b XA[i][b] XB[j][b] sum_{k in block b} A[i][k] B[j][k], 0 )
 *
 * Arguments
 *   A    device pointer, M rows of K elements (row-major, element format fmt;
 *        E2M1 rows are K / 2 bytes, element k in the low nibble of byte k / 2
 *        when k is even, the high nibble when odd).
 *   SA   device pointer, M x (K / 32) E8M0 bytes, row-major.
 *   B    device pointer, N rows of K elements: B is stored (N, K), the
 *        transposed layout of gemm_relu's transB = 1.
 *   SB   device pointer, N x (K / 32) E8M0 bytes, row-major.
 *   C    device pointer, M x N row-major, out_dtype; overwritten.
 *   M, N, K   >= 0, <= INT32_MAX; K a multiple of 32 (whole scale blocks).
 *   fmt  GEMM_RELU_MX_E4M3, GEMM_RELU_MX_E5M2 or GEMM_RELU_MX_E2M1.
 *   out_dtype  GEMM_RELU_F16, GEMM_RELU_BF16 or GEMM_RELU_F32.
 *   stream     a hipStream_t, or NULL.
 *
 * Numerics: each block product is formed on the scaled matrix units and summed
 * in fp32 (order unspecified); ReLU and rounding as for gemm_relu.
 * Ownership, execution and errors as for gemm_relu (EINVAL also for K not a
 * multiple of 32, an unknown fmt, or C overlapping A, B, SA or SB;
 * EUNSUPPORTED when K exceeds 2^22 storage bytes per row).
 */
int gemm_relu_mx(const void* A, const void* SA, const void* B, const void* SB, void* C,
                 int64_t M, int64_t N, int64_t K, int fmt, int out_dtype, void* stream);

/* Configuration name gemm_relu_mx would launch (as gemm_relu_plan). */
const char* gemm_relu_mx_plan(const void* A, const void* SA, const void* B, const void* SB,
                              const void* C, int64_t M, int64_t N, int64_t K, int fmt,
                              int out_dtype);

/*
 * gemm_relu_sp — the 2:4 structured-sparse product: the "2:4 structured-sparse
 * tensor core (T.gemm_sp)" item of the §4.1 timeline of page "TileLang：GPU/NPU
 * 通用算子 DSL", whose A
 * arrives compressed together with its metadata (page "从 TVM 到 TileLang…",
 * §四).  Every row of A is cut along K into groups of 4 consecutive elements
 * with at most two non-zeros; the caller passes them compressed:
 *
 *   As   device pointer, M x (K / 2) row-major, in_dtype: As[i][2q] and
 *        As[i][2q + 1] are the two stored values of group q of row i (zeros
 *        where the group has fewer non-zeros).
 *   E    device pointer, metadata bytes, blocked by 64 columns of K:
 *        ceil(K / 64) blocks, each M x 8 bytes row-major.  Group q of row i is
 *        nibble q % 2 (the low nibble for even q) of byte (q % 16) / 2 of row
 *        i's 8 bytes in block q / 16; the nibble is p0 | p1 << 2, the positions
 *        (0..3, p0 < p1) inside the group of As[i][2q] and As[i][2q + 1].
 *        Nibbles of groups past K are ignored.  A nibble with p0 >= p1 gives an
 *        unspecified result (the library does not read E on the host).
 *   B, C, transB, stream   as for gemm_relu (B dense (K, N) or stored (N, K)).
 *   M, N, K    >= 0, <= INT32_MAX; K a multiple of 4 (whole groups).
 *   in_dtype   GEMM_RELU_F16 or GEMM_RELU_BF16 (As and B share it).
 *   out_dtype  GEMM_RELU_F16, GEMM_RELU_BF16 or GEMM_RELU_F32.
 *
 *   C[i][j] = max( sum_q As[i][2q] opB[4q + p0][j] + As[i][2q + 1] opB[4q + p1][j], 0 )
 *
 * Numerics: products summed in fp32 on the sparse matrix units (order
 * unspecified); ReLU and rounding as for gemm_relu.  Ownership and execution as
 * for gemm_relu.  Errors: EINVAL for bad sizes, K not a multiple of 4, an
 * unknown code, a NULL or misaligned pointer (As, B 2-byte aligned; C to its
 * element), or C overlapping As, E or B; EUNSUPPORTED when K > 2^22, N > 2^24,
 * or B is stored (K, N) with N < 256; EHIP as for gemm_relu.
 */
int gemm_relu_sp(const void* As, const void* E, const void* B, void* C, int64_t M, int64_t N,
                 int64_t K, int in_dtype, int out_dtype, int transB, void* stream);

/* Configuration name gemm_relu_sp would launch (as gemm_relu_plan). */
const char* gemm_relu_sp_plan(const void* As, const void* E, const void* B, const void* C,
                              int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype,
                              int transB);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_RELU_H */
