// Fused dense GEMM + ReLU for CDNA4 (gfx950): C = max(A·op(B), 0).
//
// The operation is the running example of page "TileLang：GPU/NPU 通用算子 DSL"
// (§3.2 GPU minimal example): a block of C is owned by one workgroup, its fp32
// accumulator is cleared, the K range is walked in BK-wide steps that stage an
// A tile and a B tile from global memory into shared memory through a
// multi-buffered pipeline, each step is contracted on the matrix units, and
// the accumulator goes through max(x, 0) and a type conversion before it is
// stored.  §3.3 of the same page adds the bf16 variant with B stored (N, K)
// (transpose_B) and an fp32 C.  Page "从 TVM 到 TileLang…", §三, adds the
// thread-block rasterisation swizzle (panel of tile rows) for L2 reuse.
//
// The same kernel takes 8-bit inputs (OCP E4M3 / E5M2): the FP8 GEMM that
// §4.1 of page "TileLang：GPU/NPU 通用算子 DSL" lists among the kernels the
// DSL covers.  The pages give it no scale factors, so it is the same
// definition over the 8-bit values.
//
// What is specific to gfx950 here (none of it is on the pages):
//   * v_mfma_f32_32x32x16_{f16,bf16}: each lane feeds 8 consecutive k of one
//     row (or column) and owns 16 fp32 results of a 32x32 block;
//     v_mfma_f32_32x32x64_f8f6f4 (8-bit inputs, no block scales): the same
//     result layout, each lane feeding 32 consecutive k;
//     v_mfma_f32_16x16x32_{f16,bf16}: each lane feeds 8 consecutive k of one of
//     16 rows (4 k groups) and owns 4 fp32 results of a 16x16 block — per MAC
//     it moves less accumulator data than the 32x32 form, and on random data
//     the power-limited chip clocks it higher;
//   * global_load_lds_dwordx4: a wave writes 64 x 16 B straight into LDS, lane
//     i at base + 16 i, with no register round trip; the XOR swizzle of the LDS
//     layout is realised by choosing which global 16 B chunk each lane fetches;
//   * ds_read_b64_tr_b16 / _b8: the LDS transpose reads that turn an
//     n-contiguous B tile into k-contiguous MFMA operands, so row-major B needs
//     no transpose pass;
//   * 256 CUs in 8 XCDs with one L2 each: workgroup w is placed on XCD w mod 8,
//     so the tile order is remapped to give each XCD a contiguous run of tiles
//     before the panel swizzle is applied.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gemm_relu_hip {

enum : int { DT_F16 = 0, DT_BF16 = 1, DT_F32 = 2, DT_F8E4M3 = 3, DT_F8E5M2 = 4 };
// Block-scaled (MX) element formats: E4M3 / E5M2 bytes, or E2M1 nibbles packed
// two per byte (even k in the low nibble).  Their K geometry is in storage
// bytes: an E2M1 row of K elements is K / 2 bytes.
enum : int { DT_MX_E4M3 = 5, DT_MX_E5M2 = 6, DT_MX_E2M1 = 7 };

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

#define GR_LDS __attribute__((address_space(3)))

struct KernelArgs {
    const unsigned char* A;   // (M, K) row-major, 16- or 8-bit elements
    const unsigned char* B;   // (K, N) row-major, or (N, K) row-major when transposed
    unsigned char* C;         // (M, N) row-major, 2- or 4-byte elements
    int M, N, K;
    int tiles_m, tiles_n;
    int panel;                // tile rows per rasterisation panel (>= 1)
    const unsigned char* SA;  // block-scaled inputs: (M, KB) E8M0 scales of A, else unused
    const unsigned char* SB;  // (N, KB) E8M0 scales of B (stored (N, K))
    int KB;                   // scale blocks per row (K elements / 32)
    int nxcd;                 // XCDs the dispatcher round-robins over (1 = no remap)
    // Stream-K configurations: workgroups [0, dp_tiles) take whole tiles; the
    // next sk_units split the K steps of the remaining tiles evenly.  ws holds
    // 2 sk_units fp32 partial tiles (BM x BN each), flags one arrival counter
    // per split tile, zero between launches.
    float* ws;
    unsigned* flags;
    int dp_tiles, sk_units;
    // Two-region grids (a last round of narrower tiles): workgroups [0, tiles1)
    // take the tiles_m x tiles_n tiles of the columns [0, n_org2); the rest take
    // the tiles_m2 x tiles_n2 tiles of the second configuration over the
    // columns [n_org2, N).  tiles1 is a multiple of nxcd.
    int tiles1;
    int tiles_m2, tiles_n2, panel2, n_org2;
    // K-split configurations: workgroup w takes part s = w div T of tile
    // w mod T (T = tiles_m tiles_n): the K steps [s split_steps, (s + 1)
    // split_steps).  Its fp32 partial tile goes to slot s T + tile of ws (BM x
    // BN floats each); flags holds one arrival counter per tile, zero between
    // launches.
    int splits, split_steps;
};

// The tiles one configuration covers inside a launch: a grid of tiles_m x
// tiles_n tiles whose first column starts at n_org.
struct Region {
    int tiles_m, tiles_n, panel, n_org;
};

// ------------------------------------------------------------------ helpers
// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4]<<14).
__host__ __device__ constexpr int waitcnt_vm(int n)
{
    return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14);
}

// Barrier that orders LDS only: waits for this wave's LDS traffic (lgkmcnt), not
// for its outstanding global loads, which keep streaming later pipeline stages.
__device__ __forceinline__ void barrier_lds()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane i's bytes land at LDS address M0 + 16 i.  Written as inline asm so that
// the compiler does not treat later LDS reads as dependent on it (it would
// otherwise drain every outstanding copy before each read); completion is
// tracked explicitly with s_waitcnt vmcnt.  `lds` must be wave-uniform.
__device__ __forceinline__ void dma16(const unsigned char* gbase, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "s_nop 0\n\t"
                 "global_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(gbase), "s"(lds)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const GR_LDS unsigned char* p)
{
    return (uint32_t)(uintptr_t)p;
}

__device__ __forceinline__ u32x4_t lds_read_b128(const GR_LDS unsigned char* p)
{
    return *reinterpret_cast<const GR_LDS u32x4_t*>(p);
}

__device__ __forceinline__ i16x4_t lds_read_tr16(const GR_LDS unsigned char* p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<GR_LDS i16x4_t*>(const_cast<GR_LDS unsigned char*>(p)));
}

__device__ __forceinline__ i32x2_t lds_read_tr8(const GR_LDS unsigned char* p)
{
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        reinterpret_cast<GR_LDS i32x2_t*>(const_cast<GR_LDS unsigned char*>(p)));
}

// f(integral_constant<int, I>) for I = B .. E-1, each I a compile-time constant.
template <int B, int E, class F> __device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Input element types and MFMA shapes.  MB is the MFMA block (32: 32x32 C
// block; 16: 16x16), NG = 64 / MB lane groups along k.  A lane's operand holds
// the OPB bytes of KMF / NG consecutive k of one row (or column): OPB / 16
// chunks of 16 bytes from a k-contiguous LDS row, or OPB / 8 transpose reads
// of TRK k rows each from an n-contiguous one.  Acc is a lane's share of one
// C block (NACC fp32 values).
template <int IN_DT, int MB = 32> struct InTraits {
    static_assert(MB == 32 || MB == 16, "MFMA block");
    static constexpr int EB = 2, KMF = MB == 32 ? 16 : 32, OPB = 16, TRK = 4;
    static constexpr int NACC = MB * MB / 64;
    static constexpr bool MX = false;
    static constexpr int EPB = 1;                // elements per storage byte (unused: 2-byte elements)
    using Op = i16x8_t;
    using Acc = std::conditional_t<MB == 32, f32x16_t, f32x4_t>;
    __device__ static Acc mfma(Op a, Op b, Acc c)
    {
        if constexpr (MB == 32) {
            if constexpr (IN_DT == DT_F16)
                return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                              __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
            else
                return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                               __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
        } else {
            if constexpr (IN_DT == DT_F16)
                return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                              __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
            else
                return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                               __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
        }
    }
    // part x (< OPB / 16) of an operand from one 16-byte LDS read
    template <int X> __device__ static void set_chunk(Op& v, u32x4_t c)
    {
        v = __builtin_bit_cast(Op, c);
    }
    // part t (< OPB / 8) of an operand from one transpose read
    __device__ static void set_tr(Op& v, int t, const GR_LDS unsigned char* p)
    {
        const i16x4_t r = lds_read_tr16(p);
        if (t == 0)
            v.lo = r;
        else
            v.hi = r;
    }
};
template <int FMT> struct InTraitsF8 {
    static constexpr int EB = 1, KMF = 64, OPB = 32, TRK = 8, NACC = 16;
    static constexpr bool MX = false;
    static constexpr int EPB = 1;
    using Op = i32x8_t;
    using Acc = f32x16_t;
    // format codes of the f8f6f4 MFMA: 0 = E4M3, 1 = E5M2; no block scales
    __device__ static Acc mfma(Op a, Op b, Acc c)
    {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, 0, 0, 0, 0);
    }
    template <int X> __device__ static void set_chunk(Op& v, u32x4_t c)
    {
        if constexpr (X == 0)
            v.lo = __builtin_bit_cast(i32x4_raw, c);
        else
            v.hi = __builtin_bit_cast(i32x4_raw, c);
    }
    __device__ static void set_tr(Op& v, int t, const GR_LDS unsigned char* p)
    {
        const i32x2_t r = lds_read_tr8(p);
        v[2 * t] = r[0];
        v[2 * t + 1] = r[1];
    }
    typedef int i32x4_raw __attribute__((ext_vector_type(4)));
};
// Block-scaled (MX) inputs on v_mfma_scale_f32_32x32x64_f8f6f4.  Each lane
// supplies, with its operand, the E8M0 scale of the 32-element block it holds
// (lane 32 g + i: block g of row / column i of the MFMA's 64-k step).  The
// geometry is in storage bytes (EPB elements per byte): a k step is KMF bytes
// of a row.  E4M3 / E5M2: the 32 bytes of lane group g are k chunks g and
// 2 + g (halves of both blocks, which is how the scaled MFMA pairs bytes with
// blocks); E2M1: the 16 bytes of lane group g are chunk g (its block).
template <int FMT> struct InTraitsMX {
    static constexpr bool MX = true;
    static constexpr int EB = 1, EPB = FMT == 4 ? 2 : 1;
    static constexpr int KMF = 64 / EPB, OPB = 32 / EPB, TRK = 8, NACC = 16;
    using Op = i32x8_t;
    using Acc = f32x16_t;
    __device__ static Acc mfma_scaled(Op a, Op b, Acc c, int scale_a, int scale_b)
    {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, 0, scale_a, 0,
                                                               scale_b);
    }
    // 16-byte chunk of lane group g, part x, k step s, within a row
    __device__ static constexpr int chunk(int s, int g, int x)
    {
        return EPB == 2 ? 2 * s + g : 4 * s + 2 * x + g;
    }
    template <int X> __device__ static void set_chunk(Op& v, u32x4_t c)
    {
        if constexpr (X == 0)
            v.lo = __builtin_bit_cast(i32x4_raw, c);
        else
            v.hi = __builtin_bit_cast(i32x4_raw, c);
    }
    __device__ static void set_tr(Op&, int, const GR_LDS unsigned char*) {}
    typedef int i32x4_raw __attribute__((ext_vector_type(4)));
};
template <int MB> struct InTraits<DT_MX_E4M3, MB> : InTraitsMX<0> {};
template <int MB> struct InTraits<DT_MX_E5M2, MB> : InTraitsMX<1> {};
template <int MB> struct InTraits<DT_MX_E2M1, MB> : InTraitsMX<4> {};
template <int MB> struct InTraits<DT_F8E4M3, MB> : InTraitsF8<0> {
    static_assert(MB == 32, "8-bit inputs use the 32x32 block");
};
template <int MB> struct InTraits<DT_F8E5M2, MB> : InTraitsF8<1> {
    static_assert(MB == 32, "8-bit inputs use the 32x32 block");
};

// Output conversion after the ReLU.  max(x, 0) is written as a select so that
// a negative (or -0) sum becomes +0.
__device__ __forceinline__ float relu(float x) { return x > 0.0f ? x : 0.0f; }

template <int OUT_DT> struct OutTraits;
template <> struct OutTraits<DT_F16> {
    static constexpr int bytes = 2;
    __device__ static unsigned short cvt(float x)
    {
        return __builtin_bit_cast(unsigned short, (_Float16)x);
    }
};
template <> struct OutTraits<DT_BF16> {
    static constexpr int bytes = 2;
    __device__ static unsigned short cvt(float x)
    {
        return __builtin_bit_cast(unsigned short, (__bf16)x);
    }
};
template <> struct OutTraits<DT_F32> {
    static constexpr int bytes = 4;
};

// ---------------------------------------------------------- configuration
template <int IN_DT_, int OUT_DT_, bool TRANS_B_, int BM_, int BN_, int BK_, int WAVES_M_,
          int WAVES_N_, int STAGES_, bool DIRECT_, bool INTERLEAVE_ = false, int MB_ = 32,
          bool PERSISTENT_ = false, bool STREAMK_ = false, bool SPLITK_ = false>
struct Cfg {
    static constexpr bool PERSISTENT = PERSISTENT_;   // tile loop over a grid of <= 1 per CU
    static constexpr bool STREAMK = STREAMK_;         // last round split along K
    static constexpr bool SPLITK = SPLITK_;           // every tile split along K into fp32 partials
    static constexpr int IN_DT = IN_DT_, OUT_DT = OUT_DT_;
    static constexpr bool TRANS_B = TRANS_B_, DIRECT = DIRECT_, INTERLEAVE = INTERLEAVE_;
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, STAGES = STAGES_;
    static constexpr int NWAVES = WAVES_M * WAVES_N;
    static constexpr int NTHREADS = 64 * NWAVES;
    static constexpr int MB = MB_;                                 // MFMA C block (32 or 16)
    static constexpr int NG = 64 / MB;                             // lane groups along k
    using In = InTraits<IN_DT, MB>;
    static constexpr int EB = In::EB;                              // bytes per input element
    static constexpr int EPC = 16 / EB;                            // elements per 16 B chunk
    static constexpr int FRAG_CH = In::OPB / 16;                   // 16 B reads per k-contiguous operand
    static constexpr int TR_READS = In::OPB / 8;                   // transpose reads per n-contiguous operand
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;   // wave tile
    static constexpr int TM = WM / MB, TN = WN / MB;               // MFMA blocks per wave
    static constexpr int KSUB = BK / In::KMF;                      // MFMA k-steps per BK step
    static constexpr int ROW_CH = BK * EB / 16;                    // 16 B chunks per k-contiguous row
    static constexpr int NROW_CH = BN * EB / 16;                   // 16 B chunks per n-contiguous row
    static constexpr int A_BYTES = BM * BK * EB;
    static constexpr int B_BYTES = BN * BK * EB;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr bool MX = In::MX;
    // Scale blocks per row per BK step (block-scaled inputs).
    static constexpr int BPS = MX ? BK * In::EPB / 32 : 1;
    // Block-scaled inputs on the interleaved pipeline keep their scales in
    // LDS: for a group of SGS steps, the 16 scale bytes of each of the tile's
    // BM + BN rows (one 16-byte copy per row), in two regions that alternate
    // by group.
    static constexpr bool MX_LDS = MX && INTERLEAVE_;
    static constexpr int SGS = MX_LDS ? 16 / BPS : 1;
    static constexpr int SC_REGION = MX_LDS ? (BM + BN) * 16 : 0;
    static constexpr int SC_COPIES = MX_LDS ? (BM + BN) / NTHREADS : 0;   // per thread per group
    // ... and a word-major copy of each group (word k of every row, rows 4
    // bytes apart), in two more regions, which the per-step reads use
    static constexpr int SC_T_REGION = SC_REGION;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES + 2 * SC_REGION + 2 * SC_T_REGION;
    static constexpr int A_CH = BM * ROW_CH;                       // 16 B chunks per stage
    static constexpr int B_CH = BN * BK * EB / 16;
    static constexpr int A_PER_THREAD = A_CH / NTHREADS;
    static constexpr int B_PER_THREAD = B_CH / NTHREADS;
    static constexpr int LOADS_PER_STAGE = A_PER_THREAD + B_PER_THREAD;  // vm ops per wave per stage

    static_assert(BM % (MB * WAVES_M) == 0 && BN % (MB * WAVES_N) == 0, "wave tiling");
    static_assert(MB == 32 || TRANS_B || (BN * EB) % 256 == 0,
                  "16x16 blocks read (K,N) B rows of whole 16-chunk bank windows");
    static_assert(BK * EB == 64 || BK * EB == 128 || BK * EB == 256, "k-contiguous rows of 64, 128 or 256 bytes");
    static_assert(KSUB >= 1 && BK % In::KMF == 0, "whole MFMA k-steps per BK step");
    static_assert(KSUB % 2 == 0 || INTERLEAVE_, "an odd k-step count needs the step-parity tags of the interleaved loop");
    static_assert(!MX || (TRANS_B && DIRECT && MB_ == 32 && (INTERLEAVE_ ? STAGES_ == 4 : STAGES_ == 2)),
                  "block-scaled inputs: B stored (N,K); the two-stage direct pipeline or the "
                  "four-stage interleaved one");
    static_assert(!MX_LDS || ((BPS == 2 || BPS == 4) && BM % NTHREADS == 0 && BN % NTHREADS == 0),
                  "LDS-staged scales: 2 or 4 blocks per step; whole A and B row sets per copy");
    static_assert(!MX_LDS || SGS >= 4, "a scale group is rearranged two steps after its copies, "
                                        "before its first read");
    static_assert(A_CH % NTHREADS == 0 && B_CH % NTHREADS == 0, "loader tiling");
    static_assert(TRANS_B || NROW_CH >= (EB == 2 ? 4 : 2), "n-contiguous B rows of at least 64 (16-bit) or 32 (8-bit) bytes");
    static_assert(STAGES >= 2 && STAGES <= 5, "stages");
    static_assert((STAGES - 2) * LOADS_PER_STAGE + SC_COPIES < 64, "vmcnt range");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity of a gfx950 CU");
    static_assert(!STREAMK_ || (INTERLEAVE_ && !MX && !PERSISTENT_),
                  "stream-K: the interleaved pipeline, unscaled inputs");
    static_assert(!SPLITK_ || (DIRECT_ && !INTERLEAVE_ && !MX && !PERSISTENT_ && !STREAMK_),
                  "K split: the plain direct pipeline, unscaled inputs");

    // Interleaved direct pipeline: the LOADS_PER_STAGE copies of the stage
    // STAGES-1 ahead are spread over the KSUB k-steps of a BK step, one per
    // scheduling region; each region also carries a share of the next
    // k-step's fragment reads and of the current k-step's MFMAs.
    static constexpr int NM = TM * TN;                          // MFMAs per k-step
    static constexpr int NR = TM * FRAG_CH + TN * (TRANS_B ? FRAG_CH : TR_READS);  // LDS read ops per k-step
    static constexpr int REGIONS = LOADS_PER_STAGE / KSUB;      // = copies per k-step
    static_assert(!INTERLEAVE || (DIRECT && STAGES >= 3), "interleave needs >= 3 direct stages");
    static_assert(!INTERLEAVE || (LOADS_PER_STAGE % KSUB == 0 && REGIONS >= 1 &&
                                  (MB == 16 || NM % REGIONS == 0)),
                  "interleave: copies split evenly over the k-steps (and, for 32x32 blocks, "
                  "MFMAs over the regions; 16x16-block tiles take NM r / R .. NM (r+1) / R)");
    // Copies issued after the last copy of stage t+1 when the wave waits for it
    // (start of the last k-step of step t) in the steady state: the whole of
    // stages t+2 .. t+S-2 and the first KSUB-1 k-steps' share of stage t+S-1
    // (plus, for LDS-staged scales, a scale group's SC_COPIES when one was
    // issued in that span; the kernel adds those at run time).
    static constexpr int STEADY_ALLOWANCE =
        (STAGES - 3) * LOADS_PER_STAGE + (KSUB - 1) * (LOADS_PER_STAGE / KSUB);
    static_assert(!INTERLEAVE || STEADY_ALLOWANCE < 64, "vmcnt range");
};

// LDS banks on gfx950: 64 banks x 4 bytes, so one cycle serves 256 bytes —
// 16 lanes of a 16-byte read, 32 lanes of an 8-byte read.  The swizzles below
// make those lane groups hit 16 distinct 16-byte bank groups.

// XOR swizzle of a k-contiguous tile row (A, or B stored (N,K)) of ROW_CH
// chunks: RPW = 16 / ROW_CH rows share one 256-byte bank window, and the
// 16 lanes that read one logical chunk of 16 consecutive rows land on
// (row mod RPW, chunk ^ swz) pairs that are all distinct.
template <int ROW_CH>
__device__ __forceinline__ int swz_krow(int r)
{
    if constexpr (ROW_CH >= 16)
        return r & 15;
    else
        return (r / (16 / ROW_CH)) % ROW_CH;
}

// XOR swizzle of an n-contiguous B row (B stored (K,N)) of NROW_CH chunks.
// A transpose read serves 32 lanes per cycle: TRK consecutive k rows x W =
// 16 / TRK consecutive chunks (16-bit: 4 rows x 4 chunks; 8-bit: 8 rows x 2
// chunks).  With RPW = 16 / NROW_CH rows sharing a 256-byte bank window (1
// when the row fills it), XOR-ing the chunk index with W ((k / RPW) mod
// (NROW_CH / W)) puts those TRK rows on disjoint chunk groups of the window.
// The swizzle repeats every TRK rows, so rows k and k + TRK share it.
//
// With 16x16 blocks (16-bit inputs, rows of >= 16 chunks) the 32 lanes are two
// k groups of one block: rows 4 t + (0..3) and 8 + 4 t + (0..3), 2 chunks each;
// XOR-ing with 2 (k mod 4) + 8 ((k / 8) mod 2) spreads those 8 rows over the 8
// chunk pairs of the window.  This swizzle repeats every 16 rows only.
template <int NROW_CH, int TRK, int MB = 32>
__device__ __forceinline__ int swz_nrow(int k)
{
    if constexpr (MB == 16) {
        static_assert(NROW_CH >= 16, "16x16 blocks: rows of >= 16 chunks");
        return 2 * (k & 3) + 8 * ((k >> 3) & 1);
    } else {
        constexpr int W = 16 / TRK;
        constexpr int WIN = NROW_CH < 16 ? NROW_CH : 16;
        constexpr int RPW = 16 / WIN;
        return W * ((k / RPW) % (WIN / W));
    }
}

// ------------------------------------------------------------ tile order
// Workgroup id -> (tile row, tile col).  First an XCD-aware remap: the
// dispatcher places workgroup w on XCD (w mod 8), so tiles are renumbered to
// give every XCD one contiguous run of the logical order.  Then a panel
// swizzle: the logical order walks a panel of `panel` tile rows column by
// column, so tiles resident together share A row panels and B column panels.
__device__ __forceinline__ void tile_coords(int wg, int tiles_m, int tiles_n, int panel, int nxcd,
                                            int& tm, int& tn)
{
    const int total = tiles_m * tiles_n;
    const int per = total / nxcd, rem = total % nxcd;
    const int xcd = wg % nxcd, local = wg / nxcd;
    const int logical = xcd < rem ? xcd * (per + 1) + local
                                  : rem * (per + 1) + (xcd - rem) * per + local;
    const int panel_tiles = panel * tiles_n;
    const int p = logical / panel_tiles;
    const int within = logical - p * panel_tiles;
    const int rows = min(panel, tiles_m - p * panel);
    tm = p * panel + within % rows;
    tn = within / rows;
}

// One stream-K piece: the K steps [kt0, kt1) (of ceil(K / BK)) of a tile that
// count pieces share.  Pieces are numbered in K order; piece p > 0 is the first
// piece of unit first + p and keeps its partial in that unit's slot 2 (first +
// p); piece 0 keeps it in slot0 (its unit's second slot when the unit began in
// an earlier tile).
struct SkPiece {
    int kt0, kt1;
    int tile;      // split-tile index (its arrival counter)
    int count;     // pieces of the tile; 1: the piece is the whole tile
    int pos;       // this piece's number
    int first;     // unit of piece 0
    int slot0;     // partial slot of piece 0
};
// A workgroup's stream-K state, kept in LDS so that none of it occupies
// registers across the main loop (which needs all of them): the current
// piece, its tile's launch-order index, and the unit's remaining steps.
struct SkState {
    SkPiece pc;
    int wg;
    int lo, hi;
    int arrived;   // the piece's arrival count, for the whole workgroup
};

// ------------------------------------------------------------- the kernel
// One output tile: the tile with launch-order index wg (see tile_coords), its
// accumulator cleared, its whole K range contracted, the ReLU epilogue stored.
// Stream-K configurations contract the piece pc of it instead; see
// gemm_relu_kernel for how a tile's pieces are combined.
template <class C>
__device__ __forceinline__ void gemm_relu_tile(const KernelArgs& args, int wg,
                                               GR_LDS unsigned char* smem,
                                               GR_LDS SkState* sk, const Region& reg)
{
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, S = C::STAGES;
    constexpr int TM = C::TM, TN = C::TN, KSUB = C::KSUB;
    constexpr int ROW_CH = C::ROW_CH, NROW_CH = C::NROW_CH;
    constexpr int APT = C::A_PER_THREAD, BPT = C::B_PER_THREAD;
    constexpr int EB = C::EB, EPC = C::EPC, FRAG_CH = C::FRAG_CH, TR_READS = C::TR_READS;
    using In = typename C::In;
    using Op = typename In::Op;

    const int M = args.M, N = args.N, K = args.K;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    int tm, tn;
    tile_coords(wg, reg.tiles_m, reg.tiles_n, reg.panel, args.nxcd, tm, tn);
    const int m0 = tm * BM;
    // (K,N) B on the direct path: the last tile column is moved back to end at N,
    // so every B chunk it copies lies inside its row.  The columns it shares with
    // its neighbour are recomputed but stored by the neighbour only (n_own is the
    // tile's first stored column): each element of C has one writer, so results
    // do not depend on which tile finishes last, even when the two tiles sum
    // their K range in different pieces.
    const int n_own = reg.n_org + tn * BN;
    const int n0 = (C::DIRECT && !C::TRANS_B) ? min(n_own, N - BN) : n_own;
    // Direct path: K / BK full steps through the copy pipeline plus, if K % BK,
    // one register-staged tail step.  Register-staged path: ceil(K / BK) steps.
    // A stream-K piece or a K-split part covers the steps [kt0, kt1) of
    // ceil(K / BK): its full steps, and the tail step if it ends the K range.
    const int ksteps = (K + BK - 1) / BK;
    const int split = C::SPLITK ? (int)blockIdx.x / (reg.tiles_m * reg.tiles_n) : 0;
    const int kt0 = C::STREAMK ? sk->pc.kt0 : C::SPLITK ? split * args.split_steps : 0;
    const int kt1 = C::STREAMK ? sk->pc.kt1 : C::SPLITK ? min(ksteps, kt0 + args.split_steps) : ksteps;
    const int nk = C::DIRECT ? max(0, min(kt1, K / BK) - kt0) : ksteps;

    // ---- loader geometry: this thread owns LDS slots q = i*NTHREADS + tid of
    // each stage region; a wave's 64 slots are contiguous (one 1 KiB DMA write).
    // For every slot, the logical (row, chunk) it holds and the byte offset of
    // that chunk's source relative to the tile's global origin.
    // Slot q of a k-contiguous region holds row q / ROW_CH, logical chunk
    // (q % ROW_CH) ^ swz; slot q of an n-contiguous B region holds k row
    // q / NROW_CH, logical chunk (q % NROW_CH) ^ swz.
    auto krow_slot = [&](int q, int& r, int& c) {
        r = q / ROW_CH;
        c = (q % ROW_CH) ^ swz_krow<ROW_CH>(r);
    };
    auto nrow_slot = [&](int q, int& k, int& c) {
        k = q / NROW_CH;
        c = (q % NROW_CH) ^ swz_nrow<NROW_CH, In::TRK, C::MB>(k);
    };
    uint32_t a_src[APT];
#pragma unroll
    for (int i = 0; i < APT; ++i) {
        int r, c;
        krow_slot(i * C::NTHREADS + tid, r, c);
        const int row = min(m0 + r, M - 1) - m0;           // clamp: finite data, output discarded
        a_src[i] = (uint32_t)row * (uint32_t)K * (uint32_t)EB + (uint32_t)c * 16u;
    }
    uint32_t b_src[BPT];
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        int r, c;
        if constexpr (C::TRANS_B) {
            krow_slot(i * C::NTHREADS + tid, r, c);
            const int row = min(n0 + r, N - 1) - n0;
            b_src[i] = (uint32_t)row * (uint32_t)K * (uint32_t)EB + (uint32_t)c * 16u;
        } else {
            nrow_slot(i * C::NTHREADS + tid, r, c);
            b_src[i] = (uint32_t)r * (uint32_t)N * (uint32_t)EB + (uint32_t)c * 16u;
        }
    }

    // origins of the tile's A rows and B columns at the first K step
    const unsigned char* a_tile = args.A + (size_t)m0 * (size_t)K * EB + (size_t)kt0 * BK * EB;
    const unsigned char* b_tile = C::TRANS_B
                                      ? args.B + (size_t)n0 * (size_t)K * EB + (size_t)kt0 * BK * EB
                                      : args.B + (size_t)n0 * EB + (size_t)kt0 * BK * (size_t)N * EB;

    // ---- direct loader: global -> LDS without registers.
    const uint32_t smem_addr = lds_addr(smem);
    auto issue_direct = [&](int t, int stage) {
        const int k0 = t * BK;
        const uint32_t sa = smem_addr + stage * C::STAGE_BYTES;
        const uint32_t sb = sa + C::A_BYTES;
        const unsigned char* ga = a_tile + (size_t)k0 * EB;
        const unsigned char* gb = C::TRANS_B ? b_tile + (size_t)k0 * EB
                                             : b_tile + (size_t)k0 * (size_t)N * EB;
        // every pipelined step lies inside K and every chunk inside its row
#pragma unroll
        for (int i = 0; i < APT; ++i) dma16(ga, a_src[i], sa + (i * C::NWAVES + wave) * 1024);
#pragma unroll
        for (int i = 0; i < BPT; ++i) dma16(gb, b_src[i], sb + (i * C::NWAVES + wave) * 1024);
    };

    // ---- register-staged loader: 16 B loads where a chunk lies inside its row
    // (any 2-byte alignment: the loads run in unaligned-access mode), element-wise
    // loads with zero fill where it crosses the end of the row or the matrix,
    // then one 16 B LDS write per chunk.  The whole step of the register-staged
    // configurations; the K tail step of the direct ones.
    u32x4_t ra[APT], rb[BPT];
    auto load_chunk = [&](const unsigned char* base, size_t row_off, int e0, int e_lim,
                          bool row_ok) -> u32x4_t {
        // EPC consecutive elements e0 .. e0+EPC-1 of one row; valid if e < e_lim.
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (!row_ok) return v;
        if (e0 + EPC <= e_lim) {
            __builtin_memcpy(&v, base + row_off + (size_t)e0 * EB, 16);
        } else if constexpr (EB == 2) {
            const unsigned short* p =
                reinterpret_cast<const unsigned short*>(base + row_off) + e0;
            unsigned short h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = (e0 + e < e_lim) ? p[e] : (unsigned short)0;
            v = u32x4_t{h[0] | ((unsigned)h[1] << 16), h[2] | ((unsigned)h[3] << 16),
                        h[4] | ((unsigned)h[5] << 16), h[6] | ((unsigned)h[7] << 16)};
        } else {
            const unsigned char* p = base + row_off + e0;
            unsigned w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (e0 + e < e_lim) w[e >> 2] |= (unsigned)p[e] << (8 * (e & 3));
            v = u32x4_t{w[0], w[1], w[2], w[3]};
        }
        return v;
    };
    // chunk of slot q of stage t: A rows m0.., transposed-B rows n0.., (K,N)-B
    // rows k0.. with columns n0..
    auto a_chunk = [&](int t, int q) -> u32x4_t {
        int r, c;
        krow_slot(q, r, c);
        return load_chunk(args.A, (size_t)(m0 + r) * (size_t)K * EB, t * BK + EPC * c, K, m0 + r < M);
    };
    auto b_chunk = [&](int t, int q) -> u32x4_t {
        int r, c;
        if constexpr (C::TRANS_B) {
            krow_slot(q, r, c);
            return load_chunk(args.B, (size_t)(n0 + r) * (size_t)K * EB, t * BK + EPC * c, K,
                              n0 + r < N);
        } else {
            nrow_slot(q, r, c);
            return load_chunk(args.B, (size_t)(t * BK + r) * (size_t)N * EB, n0 + EPC * c, N,
                              t * BK + r < K);
        }
    };
    auto load_staged = [&](int t) {
#pragma unroll
        for (int i = 0; i < APT; ++i) ra[i] = a_chunk(t, i * C::NTHREADS + tid);
#pragma unroll
        for (int i = 0; i < BPT; ++i) rb[i] = b_chunk(t, i * C::NTHREADS + tid);
    };
    auto store_staged = [&](int stage) {
        GR_LDS unsigned char* sa = smem + stage * C::STAGE_BYTES;
        GR_LDS unsigned char* sb = sa + C::A_BYTES;
#pragma unroll
        for (int i = 0; i < APT; ++i)
            *reinterpret_cast<GR_LDS u32x4_t*>(sa + (i * C::NTHREADS + tid) * 16) = ra[i];
#pragma unroll
        for (int i = 0; i < BPT; ++i)
            *reinterpret_cast<GR_LDS u32x4_t*>(sb + (i * C::NTHREADS + tid) * 16) = rb[i];
    };

    // one chunk at a time (load, then LDS write): few live registers, for the
    // single K-tail step of the direct configurations
    auto fill_staged = [&](int t, int stage) {
        GR_LDS unsigned char* sa = smem + stage * C::STAGE_BYTES;
        GR_LDS unsigned char* sb = sa + C::A_BYTES;
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int q = i * C::NTHREADS + tid;
            *reinterpret_cast<GR_LDS u32x4_t*>(sa + q * 16) = a_chunk(t, q);
        }
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            const int q = i * C::NTHREADS + tid;
            *reinterpret_cast<GR_LDS u32x4_t*>(sb + q * 16) = b_chunk(t, q);
        }
    };

    // ---- fragment read geometry (per lane, relative to a stage's A / B region).
    const int wave_m = wave / C::WAVES_N, wave_n = wave % C::WAVES_N;
    const int wm0 = wave_m * C::WM, wn0 = wave_n * C::WN;
    constexpr int MB = C::MB, NG = C::NG;
    const int lr = lane % MB, g = lane / MB;     // row (column) of the block, k group
    // k-contiguous rows: for k-step s the lane reads row (w0 + MB i + lr),
    // chunks (NG s + g) FRAG_CH + x, x < FRAG_CH (its KMF / NG consecutive k;
    // block-scaled inputs place their chunks by the scaled MFMA's blocks).
    auto chunk_of = [&](int s, int x) {
        if constexpr (C::MX)
            return In::chunk(s, g, x);
        else
            return (NG * s + g) * FRAG_CH + x;
    };
    uint32_t a_rd[KSUB][FRAG_CH];
#pragma unroll
    for (int s = 0; s < KSUB; ++s)
#pragma unroll
        for (int x = 0; x < FRAG_CH; ++x) {
            const int r = wm0 + lr;
            a_rd[s][x] = (uint32_t)(r * BK * EB + ((chunk_of(s, x) ^ swz_krow<ROW_CH>(r)) * 16));
        }
    // (K,N) B offsets per block j and transpose read t (per t only where the
    // swizzle does not repeat every TRK rows: 16x16 blocks)
    constexpr int B_RD_T = C::TRANS_B ? FRAG_CH : (MB == 16 ? TR_READS : 1);
    uint32_t b_rd[C::TRANS_B ? KSUB : TN][B_RD_T];
    if constexpr (C::TRANS_B) {
#pragma unroll
        for (int s = 0; s < KSUB; ++s)
#pragma unroll
            for (int x = 0; x < FRAG_CH; ++x) {
                const int r = wn0 + lr;
                b_rd[s][x] = (uint32_t)(r * BK * EB + ((chunk_of(s, x) ^ swz_krow<ROW_CH>(r)) * 16));
            }
    } else {
        // Transpose reads: 16-lane group h holds k group gk and n-half nh of an
        // MFMA block (32x32: gk = h / 2, nh = h % 2; 16x16: gk = h, nh = 0);
        // each read covers TRK k rows, LPR lanes per row each supplying 8
        // bytes.  Lane i16 supplies row (KMF / NG) gk + i16 / LPR (+ TRK t +
        // KMF s) and the 8 bytes from column 16 nh + (i16 % LPR) (8 / EB) of
        // the block, and receives the TRK k values of column 16 nh + i16.
        constexpr int TRK = In::TRK, LPR = 16 / TRK;
        const int h = lane >> 4, i16 = lane & 15;
        const int gk = MB == 32 ? (h >> 1) : h, nh = MB == 32 ? (h & 1) : 0;
        const int kk = (In::KMF / NG) * gk + i16 / LPR;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int t = 0; t < B_RD_T; ++t) {
                const int n = wn0 + MB * j + 16 * nh + (i16 % LPR) * (8 / EB);
                const int k = kk + t * TRK;
                const int phys = ((n * EB) >> 4) ^ swz_nrow<NROW_CH, TRK, MB>(k);
                b_rd[j][t] = (uint32_t)(k * BN * EB + phys * 16 + ((n * EB) & 15));
            }
    }

    using Acc = typename In::Acc;
    constexpr int NACC = In::NACC;
    Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < NACC; ++r) acc[i][j][r] = 0.0f;

    // Fragments of one MFMA k-step: TM A blocks and TN B blocks of MB x (KMF).
    struct Frags {
        Op a[TM], b[TN];
    };
    // One LDS read op q of k-step s: the first TM FRAG_CH read A block
    // q / FRAG_CH, part q % FRAG_CH; the rest read B block j (transposed B:
    // FRAG_CH 16-byte reads; (K,N) B: TR_READS transpose reads of TRK k rows).
    auto read_op = [&](int stage, int s, int q, Frags& f) {
        const GR_LDS unsigned char* sa = smem + stage * C::STAGE_BYTES;
        const GR_LDS unsigned char* sb = sa + C::A_BYTES;
        constexpr int QA = TM * FRAG_CH;
        if (q < QA) {
            const int i = q / FRAG_CH, x = q % FRAG_CH;
            const u32x4_t v = lds_read_b128(sa + a_rd[s][x] + i * MB * BK * EB);
            if (x == 0)
                In::template set_chunk<0>(f.a[i], v);
            else
                In::template set_chunk<1>(f.a[i], v);
        } else if constexpr (C::TRANS_B) {
            const int j = (q - QA) / FRAG_CH, x = (q - QA) % FRAG_CH;
            const u32x4_t v = lds_read_b128(sb + b_rd[s][x] + j * MB * BK * EB);
            if (x == 0)
                In::template set_chunk<0>(f.b[j], v);
            else
                In::template set_chunk<1>(f.b[j], v);
        } else {
            const int j = (q - QA) / TR_READS, t = (q - QA) % TR_READS;
            const uint32_t off = B_RD_T == 1 ? b_rd[j][0] + t * In::TRK * BN * EB
                                             : b_rd[j][B_RD_T == 1 ? 0 : t];
            In::set_tr(f.b[j], t, sb + off + s * In::KMF * BN * EB);
        }
    };
    auto read_frags = [&](int stage, int s, Frags& f) {
#pragma unroll
        for (int q = 0; q < C::NR; ++q) read_op(stage, s, q, f);
    };
    // Operands swapped (B block as the MFMA's first source) so that each lane
    // ends up owning 4 consecutive n of one output row.  B blocks in snake
    // order (backwards for odd i), so one operand is unchanged from each MFMA
    // to the next.
    auto mma = [&](const Frags& f) {
        if constexpr (!C::MX) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int jj = 0; jj < TN; ++jj) {
                    const int j = (i & 1) ? TN - 1 - jj : jj;
                    acc[i][j] = In::mfma(f.b[j], f.a[i], acc[i][j]);
                }
        }
    };

    // ---- block scales (block-scaled inputs only).  For one BK step the lane
    // keeps the E8M0 scales of its TM rows of A and TN rows of B: BPS blocks
    // per row, WPS words of 4.  k-step s uses block 2 s + g of the step.
    constexpr int BPS = C::BPS;
    constexpr int WPS = (BPS + 3) / 4;
    constexpr int NSR = C::MX ? TM + TN : 1;
    uint32_t sc_cur[NSR][WPS], sc_nxt[NSR][WPS];
    int sc_row[NSR];
    if constexpr (C::MX) {
#pragma unroll
        for (int i = 0; i < TM; ++i) sc_row[i] = min(m0 + wm0 + MB * i + lr, M - 1);
#pragma unroll
        for (int j = 0; j < TN; ++j) sc_row[TM + j] = min(n0 + wn0 + MB * j + lr, N - 1);
    }
    auto scale_base = [&](int q, int t) {
        return (q < TM ? args.SA : args.SB) + (size_t)sc_row[q] * (size_t)args.KB + (size_t)t * BPS;
    };
    // scales of full step t (its blocks lie inside every row)
    auto load_scales = [&](int t, uint32_t (&dst)[NSR][WPS]) {
#pragma unroll
        for (int q = 0; q < NSR; ++q)
#pragma unroll
            for (int w = 0; w < WPS; ++w) __builtin_memcpy(&dst[q][w], scale_base(q, t) + 4 * w, 4);
    };
    // scales of the partial tail step: blocks past the row read as 2^0
    auto load_scales_tail = [&](int t, uint32_t (&dst)[NSR][WPS]) {
        const int left = args.KB - t * BPS;
#pragma unroll
        for (int q = 0; q < NSR; ++q)
#pragma unroll
            for (int w = 0; w < WPS; ++w) {
                uint32_t v = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int blk = 4 * w + b;
                    const uint32_t e = blk < left ? scale_base(q, t)[blk] : 127u;
                    v |= e << (8 * b);
                }
                dst[q][w] = v;
            }
    };
    auto mma_scaled = [&](const Frags& f, int s) {
        if constexpr (C::MX) {
            const int sh = 16 * (s & 1) + 8 * g;      // byte of block 2 s + g in word s / 2
            int sa[TM], sb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) sa[i] = (int)(sc_cur[i][s >> 1] >> sh);
#pragma unroll
            for (int j = 0; j < TN; ++j) sb[j] = (int)(sc_cur[TM + j][s >> 1] >> sh);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = In::mfma_scaled(f.b[j], f.a[i], acc[i][j], sb[j], sa[i]);
        }
    };
    auto contract = [&](const Frags& f, int s) {
        if constexpr (C::MX)
            mma_scaled(f, s);
        else
            mma(f);
    };

    Frags fr[2];
    if constexpr (C::INTERLEAVE) {
        constexpr int R = C::REGIONS, NM = C::NM, NR = C::NR, LS = C::LOADS_PER_STAGE / KSUB;
        // one copy (index l of the stage's LOADS_PER_STAGE) of stage t into its buffer
        auto issue_one = [&](int t, int stage, int l) {
            const int k0 = t * BK;
            const uint32_t sa = smem_addr + stage * C::STAGE_BYTES;
            const uint32_t sb = sa + C::A_BYTES;
            const unsigned char* ga = a_tile + (size_t)k0 * EB;
            const unsigned char* gb = C::TRANS_B ? b_tile + (size_t)k0 * EB
                                                 : b_tile + (size_t)k0 * (size_t)N * EB;
            if (l < APT)
                dma16(ga, a_src[l], sa + (l * C::NWAVES + wave) * 1024);
            else
                dma16(gb, b_src[l - APT], sb + ((l - APT) * C::NWAVES + wave) * 1024);
        };

        // ---- block scales (block-scaled inputs), staged in LDS by groups of
        // SGS steps: group G holds, for each of the tile's BM + BN rows (A rows
        // then B rows, 16 bytes apart), the row's scale bytes from block
        // off(G) on, in region G mod 2.  off(G) is 16 G except for a last,
        // partial group, which is moved back to end inside the row (rounded
        // down to whole steps).  Group G+1 is copied at the first step of
        // group G: its region was last read for step SGS G - 1, during step
        // SGS G - 2, and every wave has passed a barrier since; it is first
        // read during step SGS (G+1) - 1, after the wait for stage SGS (G+1),
        // whose copies are issued later than the group's.  Each lane reads its
        // step's scale of every A and B row it multiplies one step ahead, into
        // one of two register sets: the byte of its own block (2 blocks per
        // step) or the row's 4-byte word, of which k-step s takes byte 2 s + g
        // (4 blocks per step).
        // The reads go to a word-major copy of the group: two steps after a
        // group's copies (the step whose wait covers them), each thread moves
        // its rows' 16 bytes into word planes (word k of row q at plane k, q * 4),
        // so a read of 32 consecutive rows is 32 consecutive words.  (Read
        // straight from the 16-byte rows, 32 rows fall on 16 bank positions:
        // measured at 8192^3, about 6 conflict cycles per read.)  The plane
        // region of group G+1 was last read for step SGS G - 1.
        constexpr int SGS = C::SGS, GC = C::SC_COPIES;
        constexpr int SC_ROWS = BM + BN;
        constexpr int NSC = C::MX_LDS ? TM + TN : 1;
        uint32_t scg_src[GC > 0 ? GC : 1];
        if constexpr (C::MX_LDS) {
#pragma unroll
            for (int i = 0; i < GC; ++i) {
                const int q = i * C::NTHREADS + tid;
                const int row = q < BM ? min(m0 + q, M - 1) : min(n0 + q - BM, N - 1);
                scg_src[i] = (uint32_t)row * (uint32_t)args.KB;
            }
        }
        auto group_off = [&](int G) { return min(16 * G, (args.KB - 16) & ~(BPS - 1)); };
        // whether step u issues the copies of a scale group
        auto group_step = [&](int u) {
            return C::MX_LDS && u >= 0 && u % SGS == 0 && SGS * (u / SGS + 1) < nk;
        };
        auto issue_group = [&](int G) {
            if constexpr (C::MX_LDS) {
                const int off = group_off(G);
                const uint32_t dst = smem_addr + S * C::STAGE_BYTES + (G & 1) * C::SC_REGION;
#pragma unroll
                for (int i = 0; i < GC; ++i) {
                    const unsigned char* src = (i * C::NTHREADS < BM ? args.SA : args.SB) + off;
                    dma16(src, scg_src[i], dst + (i * C::NWAVES + wave) * 1024);
                }
            }
        };
        GR_LDS unsigned char* const sc_raw = smem + S * C::STAGE_BYTES;
        GR_LDS unsigned char* const sc_planes = sc_raw + 2 * C::SC_REGION;
        auto rearrange_group = [&](int G) {
            if constexpr (C::MX_LDS) {
                const GR_LDS unsigned char* raw = sc_raw + (G & 1) * C::SC_REGION;
                GR_LDS unsigned char* pl = sc_planes + (G & 1) * C::SC_T_REGION;
#pragma unroll
                for (int i = 0; i < GC; ++i) {
                    const int q = i * C::NTHREADS + tid;
                    const u32x4_t v = lds_read_b128(raw + q * 16);
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        *reinterpret_cast<GR_LDS uint32_t*>(pl + k * SC_ROWS * 4 + q * 4) = v[k];
                }
            }
        };
        // Reads are whole words; the step's first block is byte sc_sub of the
        // word, and the lane shifts its byte down at use.
        const int sc_a = (wm0 + lr) * 4, sc_b = (BM + wn0 + lr) * 4;
        uint32_t scv[2][NSC];
        int sc_sub[2] = {0, 0};
        auto read_scales = [&](int t, auto set_tag) {
            if constexpr (C::MX_LDS) {
                constexpr int SET = decltype(set_tag)::value;
                const int G = t / SGS;
                const int first = BPS * t - group_off(G);       // byte of the step's first block
                const GR_LDS unsigned char* pl = sc_planes + (G & 1) * C::SC_T_REGION +
                                                 (first >> 2) * SC_ROWS * 4;
                sc_sub[SET] = first & 3;
#pragma unroll
                for (int q = 0; q < NSC; ++q) {
                    const GR_LDS unsigned char* p =
                        pl + (q < TM ? sc_a + 4 * MB * q : sc_b + 4 * MB * (q - TM));
                    scv[SET][q] = *reinterpret_cast<const GR_LDS uint32_t*>(p);
                }
            }
        };
        // MFMA p of k-step s: B block j = p / TM against A block i, which runs
        // up the column for even j and down it for odd j, so the A operand is
        // unchanged from one MFMA to the next where j steps (scales from
        // register set SET for block-scaled inputs).  On random data the
        // power-limited clock is slightly higher with fewer operand changes
        // between consecutive MFMAs.
        auto mfma_op = [&](const Frags& f, int p, int s, auto set_tag) {
            const int j = p / TM, i = (j & 1) ? TM - 1 - p % TM : p % TM;
            if constexpr (C::MX) {
                constexpr int SET = decltype(set_tag)::value;
                // block 2 s + g of the step (the MFMA reads the low byte)
                const int sh = 8 * (sc_sub[SET] + 2 * s + g);
                const int sa_v = (int)(scv[SET][i] >> sh);
                const int sb_v = (int)(scv[SET][TM + j] >> sh);
                acc[i][j] = In::mfma_scaled(f.b[j], f.a[i], acc[i][j], sb_v, sa_v);
            } else {
                acc[i][j] = In::mfma(f.b[j], f.a[i], acc[i][j]);
            }
        };

        // Prologue: scale group 0, then stages 0 .. S-2.
        if (C::MX_LDS && nk > 0) issue_group(0);
#pragma unroll
        for (int st = 0; st < S - 1; ++st)
            if (st < nk) issue_direct(st, st);
        if (nk > 0) {
            if (nk - 1 >= S - 2)
                __builtin_amdgcn_s_waitcnt(waitcnt_vm((S - 2) * C::LOADS_PER_STAGE));
            else
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            barrier_lds();
            if constexpr (C::MX_LDS) {
                rearrange_group(0);
                barrier_lds();
            }
            read_scales(0, std::integral_constant<int, 0>{});
#pragma unroll
            for (int q = 0; q < NR; ++q) read_op(0, 0, q, fr[0]);
        }
        // One BK step.  STEADY: the stage S-1 ahead exists, so the step needs
        // no run-time checks.  PARITY = t mod 2: with an odd number of k-steps
        // per BK step the two fragment sets swap roles from one step to the
        // next (k-step s of step t contracts set (t KSUB + s) mod 2).  SLOT =
        // t mod S (block-scaled inputs: the scale ring).
        // RUN (block-scaled inputs): the step's position in an unrolled run of
        // SGS steady steps that starts a scale group, or -1 for a step whose
        // group duties are decided at run time.  In a run they are fixed at
        // compile time and taken unconditionally (a group past the last one
        // copies and rearranges clamped, in-bounds bytes nobody reads), so the
        // run has no branches for the compiler to move MFMAs across.
        auto step = [&](int t, auto steady_tag, auto parity_tag, auto run_tag) {
            constexpr bool STEADY = decltype(steady_tag)::value;
            constexpr int PARITY = decltype(parity_tag)::value;
            constexpr int RUN = decltype(run_tag)::value;
            const int stage = t % S;
            const bool loads = STEADY || t + S - 1 < nk;
            const int ld_stage = (t + S - 1) % S;
            const int ld_k0 = (t + S - 1) * BK;
            const unsigned char* ga = a_tile + (size_t)ld_k0 * EB;
            const unsigned char* gb = C::TRANS_B ? b_tile + (size_t)ld_k0 * EB
                                                 : b_tile + (size_t)ld_k0 * (size_t)N * EB;
            const uint32_t lsa = smem_addr + ld_stage * C::STAGE_BYTES;
            const uint32_t lsb = lsa + C::A_BYTES;
            // a scale group's copies issued after stage t+1's, before this
            // step's wait: by the previous step, or by this one when the wait
            // is not at its top
            const bool group_after = RUN >= 0 ? (RUN == 1 || (KSUB > 1 && RUN == 0))
                                              : (group_step(t - 1) || (KSUB > 1 && group_step(t)));
            const bool group_now = RUN >= 0 ? RUN == 0 : group_step(t);
            const bool rearrange_now = RUN >= 0 ? RUN == 2 : (t % SGS == 2 && group_step(t - 2));
#pragma unroll
            for (int s = 0; s < KSUB; ++s) {
                const bool last = s + 1 == KSUB;
                if (last && (STEADY || t + 1 < nk)) {
                    if (!loads)
                        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
                    else if (C::MX_LDS && group_after)
                        __builtin_amdgcn_s_waitcnt(waitcnt_vm(C::STEADY_ALLOWANCE + GC));
                    else
                        __builtin_amdgcn_s_waitcnt(waitcnt_vm(C::STEADY_ALLOWANCE));
                    barrier_lds();
                }
                if constexpr (C::MX_LDS)
                    if (s == 0 && group_now) issue_group(t / SGS + 1);
                const bool reads = !last || STEADY || t + 1 < nk;
                const int rd_stage = last ? (t + 1) % S : stage;
                const int rd_s = last ? 0 : s + 1;
                if constexpr (C::MX_LDS) {
                    // the group copied two steps ago has landed (this step's
                    // wait covers it): rearrange it before its first read,
                    // which comes at least one barrier later
                    if (last && rearrange_now) rearrange_group(t / SGS + 1);
                    if (last && reads) read_scales(t + 1, std::integral_constant<int, 1 - PARITY>{});
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    __builtin_amdgcn_sched_barrier(0);
                    const int l = s * LS + r;
                    if constexpr (STEADY) {
                        if (l < APT)
                            dma16(ga, a_src[l], lsa + (l * C::NWAVES + wave) * 1024);
                        else
                            dma16(gb, b_src[l - APT], lsb + ((l - APT) * C::NWAVES + wave) * 1024);
                    } else {
                        if (loads) issue_one(t + S - 1, ld_stage, l);
                    }
                    if (reads) {
#pragma unroll
                        for (int q = r * NR / R; q < (r + 1) * NR / R; ++q)
                            read_op(rd_stage, rd_s, q, fr[(PARITY * KSUB + s + 1) & 1]);
                    }
#pragma unroll
                    for (int p = r * NM / R; p < (r + 1) * NM / R; ++p)
                        mfma_op(fr[(PARITY * KSUB + s) & 1], p, s, parity_tag);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        // steady steps: stage t+S-1 < nk
        const int t_steady = max(0, nk - (S - 1));
        using Steady = std::integral_constant<bool, true>;
        using Checked = std::integral_constant<bool, false>;
        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        using NoRun = std::integral_constant<int, -1>;
        if constexpr (KSUB % 2 == 0 && !C::MX_LDS) {
            for (int t = 0; t < t_steady; ++t) step(t, Steady{}, P0{}, NoRun{});
            for (int t = t_steady; t < nk; ++t) step(t, Checked{}, P0{}, NoRun{});
        } else {
            // steps in pairs, so that every step's parity (fragment sets, and
            // the scale register sets) is known at compile time; a steady
            // step left over before the checked ones runs checked
            int t = 0;
            if constexpr (C::MX_LDS) {
                // whole scale groups of steady steps, unrolled (SGS is even,
                // so parities alternate within a run)
                for (; t + SGS - 1 < t_steady; t += SGS)
                    static_for<0, SGS>([&](auto k_tag) {
                        constexpr int k = decltype(k_tag)::value;
                        step(t + k, Steady{}, std::integral_constant<int, k % 2>{}, k_tag);
                    });
            }
            if constexpr (C::MB == 16 && !C::MX) {
                // 16x16 blocks (one MFMA k step per BK step, 8 x 8 blocks a
                // wave): steady steps with one fragment set, reloaded in place.
                // Fragment sets alternating by step parity need the loop
                // unrolled by two steps, and the register allocator then moves
                // the 64 small accumulators around the loop; a second set
                // copied into the first costs 64 moves a step.  Instead the
                // step's 64 MFMAs run as two halves, all A blocks against B
                // blocks 0..3 and then against B blocks 4..7 (rows of A in
                // pairs, snake order inside a pair), and each fragment is
                // read for the next step right after its last use in this
                // one: B 0..3 after the first half, A blocks 2k, 2k+1 after
                // region 4 + k, B 4..7 at the end.  Every read then has at
                // least four regions (32 MFMAs) before its first use.
                // Narrower tiles (TN = 6: 256 x 192; TN = 3: waves of 128 x 48)
                // keep the eight regions, with TN / 2 B blocks in the first half
                // and the rest in the second, and one copy in each of the first
                // LOADS_PER_STAGE regions.  With TN = 3 every read still has
                // at least three regions (six MFMAs) before its first use.
                static_assert(TM == 8 && TN >= 2 && TN <= 8 && KSUB == 1 &&
                                  C::LOADS_PER_STAGE <= 8,
                              "in-place 16x16 steps: 8 x TN blocks, at most one copy per region");
                constexpr int QA = TM * FRAG_CH;
                constexpr int QB = C::TRANS_B ? FRAG_CH : TR_READS;     // reads per B block
                constexpr int HB0 = TN / 2, HB1 = TN - HB0;               // B blocks per half
                for (; t < t_steady; ++t) {
                    const int ld_stage = (t + S - 1) % S;
                    const int ld_k0 = (t + S - 1) * BK;
                    const unsigned char* ga = a_tile + (size_t)ld_k0 * EB;
                    const unsigned char* gb = C::TRANS_B ? b_tile + (size_t)ld_k0 * EB
                                                         : b_tile + (size_t)ld_k0 * (size_t)N * EB;
                    const uint32_t lsa = smem_addr + ld_stage * C::STAGE_BYTES;
                    const uint32_t lsb = lsa + C::A_BYTES;
                    const int rd_stage = (t + 1) % S;
                    // stage t+1 has landed (this wave's copies, then the
                    // barrier for the others'), and every wave is past its reads
                    // of the buffer the copies below refill: those reads (stage
                    // t-1, issued during step t-2) fed MFMAs of step t-1, so they
                    // have completed.  No LDS fence: it would wait for this
                    // wave's just-issued reads of stage t+1 as well.  The
                    // memory clobber keeps the compiler from moving LDS accesses
                    // across the barrier.
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm(C::STEADY_ALLOWANCE));
                    asm volatile("s_barrier" ::: "memory");
                    static_for<0, 8>([&](auto r_tag) {
                        constexpr int r = decltype(r_tag)::value;
                        __builtin_amdgcn_sched_barrier(0);
                        if constexpr (r < APT)
                            dma16(ga, a_src[r], lsa + (r * C::NWAVES + wave) * 1024);
                        else if constexpr (r < C::LOADS_PER_STAGE)
                            dma16(gb, b_src[r - APT], lsb + ((r - APT) * C::NWAVES + wave) * 1024);
                        constexpr int half = r / 4, i0 = 2 * (r % 4);
                        constexpr int j0 = half ? HB0 : 0, hb = half ? HB1 : HB0;
#pragma unroll
                        for (int di = 0; di < 2; ++di)
#pragma unroll
                            for (int jj = 0; jj < hb; ++jj) {
                                const int i = i0 + di;
                                const int j = j0 + (di ? hb - 1 - jj : jj);
                                acc[i][j] = In::mfma(fr[0].b[j], fr[0].a[i], acc[i][j]);
                            }
                        if constexpr (r == 3 || r == 7) {
#pragma unroll
                            for (int q = QA + j0 * QB; q < QA + (j0 + hb) * QB; ++q)
                                read_op(rd_stage, 0, q, fr[0]);
                        }
                        if constexpr (r >= 4) {
#pragma unroll
                            for (int q = i0 * FRAG_CH; q < (i0 + 2) * FRAG_CH; ++q)
                                read_op(rd_stage, 0, q, fr[0]);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    });
                }
            }
            for (; t + 1 < t_steady; t += 2) {
                step(t, Steady{}, P0{}, NoRun{});
                step(t + 1, Steady{}, P1{}, NoRun{});
            }
            for (; t + 1 < nk; t += 2) {
                step(t, Checked{}, P0{}, NoRun{});
                step(t + 1, Checked{}, P1{}, NoRun{});
            }
            if (t < nk) step(t, Checked{}, P0{}, NoRun{});
        }
    } else if constexpr (C::DIRECT) {
        // Pipeline: S-1 stages in flight ahead of the one being contracted.
        // At the last k-step of stage t the wave waits for stage t+1, meets the
        // others at a barrier (which also retires every read of stage t, so its
        // buffer may be refilled), and starts reading stage t+1 while the last
        // MFMAs of stage t run.
        // Block-scaled inputs: step t+1's scales are loaded at the top of step
        // t, before its copies, so the wait for stage t+1 covers them too.
        if constexpr (C::MX)
            if (nk > 0) load_scales(0, sc_cur);
#pragma unroll
        for (int st = 0; st < S - 1; ++st)
            if (st < nk) issue_direct(st, st);
        if (nk > 0) {
            if (nk - 1 >= S - 1)
                __builtin_amdgcn_s_waitcnt(waitcnt_vm((S - 2) * C::LOADS_PER_STAGE));
            else
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            barrier_lds();
            read_frags(0, 0, fr[0]);
        }
        for (int t = 0; t < nk; ++t) {
            const int stage = t % S;
            if constexpr (C::MX)
                if (t + 1 < nk) load_scales(t + 1, sc_nxt);
            if (t + S - 1 < nk) issue_direct(t + S - 1, (t + S - 1) % S);
#pragma unroll
            for (int s = 0; s < KSUB; ++s) {
                if (s + 1 < KSUB) {
                    read_frags(stage, s + 1, fr[(s + 1) & 1]);
                } else if (t + 1 < nk) {
                    // stages issued after t+1: t+2 .. min(t+S-1, nk-1)
                    if (nk - 2 - t >= S - 2)
                        __builtin_amdgcn_s_waitcnt(waitcnt_vm((S - 2) * C::LOADS_PER_STAGE));
                    else
                        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
                    barrier_lds();
                    read_frags((t + 1) % S, 0, fr[(s + 1) & 1]);
                }
                contract(fr[s & 1], s);
            }
            if constexpr (C::MX)
                if (t + 1 < nk) {
#pragma unroll
                    for (int q = 0; q < NSR; ++q)
#pragma unroll
                        for (int w = 0; w < WPS; ++w) sc_cur[q][w] = sc_nxt[q][w];
                }
        }
    }
    if constexpr (C::DIRECT) {
        // K tail (K % BK != 0): one register-staged step with element-wise zero
        // fill past K, after every wave has left the copy ring.
        if (K % BK != 0 && kt1 > K / BK) {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            barrier_lds();
            if constexpr (C::MX) load_scales_tail(nk, sc_cur);
            fill_staged(kt0 + nk, 0);
            barrier_lds();
            read_frags(0, 0, fr[0]);
#pragma unroll
            for (int s = 0; s < KSUB; ++s) {
                if (s + 1 < KSUB) read_frags(0, s + 1, fr[(s + 1) & 1]);
                contract(fr[s & 1], s);
            }
        }
    } else {
        if (nk > 0) {
            load_staged(0);
            store_staged(0);
        }
        for (int t = 0; t < nk; ++t) {
            barrier_lds();
            if (t + 1 < nk) load_staged(t + 1);
            read_frags(t & 1, 0, fr[0]);
#pragma unroll
            for (int s = 0; s < KSUB; ++s) {
                if (s + 1 < KSUB) read_frags(t & 1, s + 1, fr[(s + 1) & 1]);
                mma(fr[s & 1]);
            }
            if (t + 1 < nk) {
                barrier_lds();
                store_staged((t + 1) & 1);
            }
        }
    }

    // ---- stream-K: a piece that is not the whole tile publishes its fp32
    // partial; the piece that arrives last at the tile's counter stores the
    // tile from the sum of all of them, read back in piece order.  (Summing
    // from memory leaves the accumulators to the matrix instructions alone:
    // vector adds into them make the compiler split them over both register
    // files and shuffle them every main-loop step.)  As for the K split below,
    // the partials are written and read as device-scope atomics and a piece
    // counts itself in only once its stores have completed, so no L2
    // write-back or invalidation is needed.  Partial layout: value e of group
    // v = (i TN + j) NQ + q of thread tid at float (4 v + e) NTHREADS + tid of
    // the slot (each dword store of a wave is 256 consecutive bytes).
    constexpr int NQ = NACC / 4;                 // 4-float groups per block
    bool from_partials = false;
    auto slot_of = [&](int p) {
        const GR_LDS SkPiece* pc = &sk->pc;
        const int s = p == 0 ? pc->slot0 : 2 * (pc->first + p);
        return args.ws + (size_t)s * (BM * BN) + tid;
    };
    if constexpr (C::STREAMK) {
        const GR_LDS SkPiece* pc = &sk->pc;
        if (pc->count > 1) {
            float* own = slot_of(pc->pos);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int q = 0; q < NQ; ++q)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            __hip_atomic_store(own + (((i * TN + j) * NQ + q) * 4 + e) * C::NTHREADS,
                                               acc[i][j][4 * q + e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            // this wave's stores have completed, then every wave's
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            asm volatile("s_barrier" ::: "memory");
            if (tid == 0)
                sk->arrived = (int)__hip_atomic_fetch_add(args.flags + pc->tile, 1u, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
            barrier_lds();
            if (sk->arrived + 1 != pc->count) return;     // a later piece completes the tile
            if (tid == 0)
                __hip_atomic_store(args.flags + pc->tile, 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            from_partials = true;
        }
    }

    // ---- K split: every part publishes its partial tile and counts itself in
    // at the tile's counter; the last to arrive adds the parts in K order (its
    // own from registers), so the sum is the same whichever part finishes
    // last, and goes on to the epilogue with it.  Parts never wait for one
    // another.  The partials are written and read as device-scope atomics
    // (each coherent across the XCDs' separate L2 caches by itself), and a
    // part counts itself in only once its stores have completed; so no L2
    // write-back or invalidation is needed, which a release / acquire pair
    // would do for the whole cache of every part's XCD.  Partial layout: value
    // e of group v = (i TN + j) NQ + q of thread tid at float (4 v + e)
    // NTHREADS + tid of the slot (each dword store of a wave is 256
    // consecutive bytes).
    if constexpr (C::SPLITK) {
        constexpr int NQS = NACC / 4, NV = TM * TN * NQS;
        const int tiles = reg.tiles_m * reg.tiles_n;
        const int tile = (int)blockIdx.x - split * tiles;
        auto slot = [&](int p) { return args.ws + ((size_t)(p * tiles + tile) * (BM * BN) + tid); };
        float* own = slot(split);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < NQS; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        __hip_atomic_store(own + (((i * TN + j) * NQS + q) * 4 + e) * C::NTHREADS,
                                           acc[i][j][4 * q + e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // this wave's stores have completed, then every wave's
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("s_barrier" ::: "memory");
        __shared__ int arrived;
        if (tid == 0)
            arrived = (int)__hip_atomic_fetch_add(args.flags + tile, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        barrier_lds();
        if (arrived + 1 != args.splits) return;     // a later part completes the tile
        if (tid == 0)
            __hip_atomic_store(args.flags + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the other parts' tiles in groups of PB, all of a group's loads in
        // flight together, then added in part order
        constexpr int PB = 4;
        f32x4_t sum[NV];
        for (int p0 = 0; p0 < args.splits; p0 += PB) {
            f32x4_t x[PB][NV];
#pragma unroll
            for (int u = 0; u < PB; ++u) {
                const int p = p0 + u;
                if (p < args.splits && p != split) {
                    const float* sp = slot(p);
#pragma unroll
                    for (int v = 0; v < NV; ++v)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            x[u][v][e] = __hip_atomic_load(sp + (4 * v + e) * C::NTHREADS, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
                }
            }
#pragma unroll
            for (int u = 0; u < PB; ++u) {
                const int p = p0 + u;
                if (p < args.splits) {
                    if (p == split) {
#pragma unroll
                        for (int i = 0; i < TM; ++i)
#pragma unroll
                            for (int j = 0; j < TN; ++j)
#pragma unroll
                                for (int q = 0; q < NQS; ++q)
                                    x[u][(i * TN + j) * NQS + q] =
                                        f32x4_t{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                                acc[i][j][4 * q + 3]};
                    }
#pragma unroll
                    for (int v = 0; v < NV; ++v) sum[v] = p == 0 ? x[u][v] : sum[v] + x[u][v];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < NQS; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] = sum[(i * TN + j) * NQS + q][e];
    }

    // ---- epilogue: ReLU on the fp32 accumulators, convert, store.
    // Lane owns C[m][n .. n+3] with m = m0 + wm0 + MB i + lr and
    // n = n0 + wn0 + MB j + 4 NG q + 4 g, for q < NACC / 4 (registers 4q .. 4q+3).
    // 16-bit C: the tile goes through the (now idle) LDS ring so that the
    // global stores are whole rows, 16 bytes per lane, instead of 8-byte
    // pieces of 32 different rows.  Those whole-row 16-byte stores are
    // non-temporal.  Row r of the staged tile keeps its 16-byte
    // chunk c at c ^ (r mod 16) (mod the row's chunk count when shorter):
    // conflict-free row reads, 2-way writes.  Otherwise (fp32 C, or a tile
    // larger than the ring): four values inside the row go out as one 8- or
    // 16-byte store (any element alignment: unaligned-access mode); a row's
    // last partial group element-wise.
    constexpr int OB = OutTraits<C::OUT_DT>::bytes;
    constexpr bool STAGED = OB == 2 && BM * BN * 2 <= C::LDS_BYTES;
    constexpr int RB = BN * 2, RCH = BN / 8;          // staged: bytes and chunks per tile row
    // chunk swizzle mask: the largest power of two <= 16 dividing RCH, less one
    // (a row of 24 chunks XORs inside aligned groups of 8)
    constexpr int XM = (RCH % 16 == 0 ? 16 : RCH % 8 == 0 ? 8 : RCH % 4 == 0 ? 4 : 1) - 1;
    auto put_group = [&](int i, int j, int q, const f32x4_t& x) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = relu(x[e]);
        if constexpr (STAGED) {
            const int r = wm0 + MB * i + lr;
            const int c = wn0 + MB * j + 4 * NG * q + 4 * g;
            unsigned short h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = OutTraits<C::OUT_DT>::cvt(v[e]);
            const u32x2_t w = {h[0] | ((unsigned)h[1] << 16), h[2] | ((unsigned)h[3] << 16)};
            *reinterpret_cast<GR_LDS u32x2_t*>(smem + r * RB + (((c >> 3) ^ (r & XM)) << 4) +
                                               (c & 7) * 2) = w;
        } else {
            const int m = m0 + wm0 + MB * i + lr;
            const int n = n0 + wn0 + MB * j + 4 * NG * q + 4 * g;
            if (m >= M || n >= N || n + 4 <= n_own) return;
            unsigned char* crow = args.C + (size_t)m * (size_t)N * OB;
            const bool whole = n >= n_own && n + 4 <= N;
            if constexpr (C::OUT_DT == DT_F32) {
                float* dst = reinterpret_cast<float*>(crow) + n;
                if (whole) {
                    const u32x4_t w = {__builtin_bit_cast(unsigned, v[0]), __builtin_bit_cast(unsigned, v[1]),
                                       __builtin_bit_cast(unsigned, v[2]), __builtin_bit_cast(unsigned, v[3])};
                    // an ordinary store: these 16-byte pieces of 32 rows per
                    // instruction need L2 to combine them into whole lines
                    // (non-temporal, 4096x7168x4096 bf16 -> fp32 ran 1.4x slower)
                    __builtin_memcpy(dst, &w, 16);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e >= n_own && n + e < N) dst[e] = v[e];
                }
            } else {
                unsigned short h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = OutTraits<C::OUT_DT>::cvt(v[e]);
                unsigned short* dst = reinterpret_cast<unsigned short*>(crow) + n;
                if (whole) {
                    const u32x2_t w = {h[0] | ((unsigned)h[1] << 16), h[2] | ((unsigned)h[3] << 16)};
                    __builtin_memcpy(dst, &w, 8);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e >= n_own && n + e < N) dst[e] = h[e];
                }
            }
        }
    };
    if constexpr (STAGED) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        barrier_lds();
    }
    auto put_acc = [&] {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const f32x4_t x = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                       acc[i][j][4 * q + 3]};
                    put_group(i, j, q, x);
                }
    };
    if constexpr (C::STREAMK) {
        if (from_partials) {
            // groups of VB: the sum p_0 + p_1 + ... of each, then its stores
            constexpr int NV = TM * TN * NQ, VB = 16;
            static_assert(NV % VB == 0, "partial load batches");
            const int count = sk->pc.count;
            auto load_batch = [&](int p, int c, f32x4_t* x) {
                const float* sp = slot_of(p);
#pragma unroll
                for (int k = 0; k < VB; ++k)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        x[k][e] = __hip_atomic_load(sp + (4 * (c + k) + e) * C::NTHREADS, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
            };
#pragma unroll
            for (int c = 0; c < NV; c += VB) {
                f32x4_t sum[VB];
                load_batch(0, c, sum);
                for (int p = 1; p < count; ++p) {
                    f32x4_t x[VB];
                    load_batch(p, c, x);
#pragma unroll
                    for (int k = 0; k < VB; ++k) sum[k] += x[k];
                }
#pragma unroll
                for (int k = 0; k < VB; ++k) {
                    const int v = c + k, b = v / NQ;
                    put_group(b / TN, b % TN, v % NQ, sum[k]);
                }
            }
        } else {
            put_acc();
        }
    } else {
        put_acc();
    }
    if constexpr (STAGED) {
        barrier_lds();
        auto store_chunk = [&](int r, int cc) {
            const int m = m0 + r, n = n0 + 8 * cc;
            if (m >= M || n >= N || n + 8 <= n_own) return;
            const u32x4_t v = *reinterpret_cast<const GR_LDS u32x4_t*>(
                smem + r * RB + ((cc ^ (r & XM)) << 4));
            unsigned short* dst = reinterpret_cast<unsigned short*>(args.C) + (size_t)m * N + n;
            if (n >= n_own && n + 8 <= N) {
                // streaming store: C is not read again, so its lines should not
                // push the next tiles' operand panels out of L2
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(dst));
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (n + e >= n_own && n + e < N)
                        dst[e] = (unsigned short)(v[e >> 1] >> (16 * (e & 1)));
            }
        };
        if constexpr (C::NTHREADS % RCH == 0) {
            // whole rows per pass: thread tid keeps chunk tid % RCH
            constexpr int ROWS_PER_PASS = C::NTHREADS / RCH;
            static_assert(BM % ROWS_PER_PASS == 0, "epilogue row passes");
            const int cc = tid % RCH;
#pragma unroll 4
            for (int r = tid / RCH; r < BM; r += ROWS_PER_PASS) store_chunk(r, cc);
        } else {
            static_assert((BM * RCH) % C::NTHREADS == 0, "epilogue chunk passes");
#pragma unroll 4
            for (int idx = tid; idx < BM * RCH; idx += C::NTHREADS) store_chunk(idx / RCH, idx % RCH);
        }
    }
}

// ------------------------------------------- persistent 16x16-block tiles
// The T.Persistent form of page "TileLang：GPU/NPU 通用算子 DSL", §3.3, for the
// 16x16-block tile: a grid of at most one workgroup per CU, workgroup w taking
// tiles w, w + G, w + 2G, ... (G = grid, a multiple of the XCD count, so every
// tile of a workgroup keeps the placement the one-tile-per-workgroup grid
// gives it).  The K steps of a workgroup's tiles form one stream through the
// stage ring: during the last S-1 steps of a tile the copies fetch the first
// S-1 steps of the next tile, and the last step's in-place fragment reloads
// read the next tile's first step, so the next tile starts without the
// pipeline's fill latency.  C goes out straight from the accumulators (the
// ring is busy with the next tile, so it cannot stage C), and the next tile's
// MFMAs start while those stores drain.
//
// Every tile lies inside the matrix: the last tile row and column are moved
// back to end at M and N, and each moved-back tile stores only the rows and
// columns its neighbours do not own, so every element of C has one writer and
// no copy is clamped.  Needs M, N >= 256 and K a multiple of 32 with at least
// S steps (plan selection checks).
template <class C>
__device__ __forceinline__ void gemm_relu_i16_persistent(const KernelArgs& args,
                                                         GR_LDS unsigned char* smem)
{
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, S = C::STAGES;
    constexpr int TM = C::TM, TN = C::TN;
    constexpr int APT = C::A_PER_THREAD, BPT = C::B_PER_THREAD, LOADS = C::LOADS_PER_STAGE;
    constexpr int ROW_CH = C::ROW_CH, NROW_CH = C::NROW_CH;
    constexpr int EB = C::EB, FRAG_CH = C::FRAG_CH, TR_READS = C::TR_READS;
    constexpr int MB = 16, NG = 4;
    using In = typename C::In;
    using Op = typename In::Op;
    using Acc = typename In::Acc;
    static_assert(C::MB == 16 && !C::MX && C::DIRECT && C::INTERLEAVE && C::KSUB == 1 && TM == 8 &&
                      TN % 2 == 0 && TN <= 8 && LOADS <= 8 && !C::STREAMK,
                  "persistent 16x16-block tile: 8 x TN blocks, one copy per region");

    const int M = args.M, N = args.N, K = args.K;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nk = K / BK;
    const int total = args.tiles_m * args.tiles_n;
    const int G = gridDim.x;
    int tile = blockIdx.x;
    if (tile >= total) return;

    // ---- copy geometry, the same for every tile (no clamped rows): slot q of
    // a k-contiguous region holds row q / ROW_CH, chunk (q % ROW_CH) ^ swz;
    // slot q of an n-contiguous B region holds k row q / NROW_CH.  Copy i of a
    // lane covers the rows of copy 0 shifted by i passes; the swizzles repeat
    // every 16 rows, so one per-lane offset (two for an n-contiguous B, whose
    // passes are 8 rows) and a scalar shift per copy locate every chunk, which
    // keeps the vector registers for the accumulators and fragments.
    constexpr int RPP = C::NTHREADS / ROW_CH;       // k-contiguous rows per copy pass
    constexpr int KPP = C::NTHREADS / NROW_CH;      // n-contiguous B rows per copy pass
    constexpr int NPAT = C::TRANS_B || KPP >= 16 ? 1 : 16 / KPP;
    static_assert(RPP % 16 == 0 && (C::TRANS_B || KPP % 16 == 0 || 16 % KPP == 0) && BPT % NPAT == 0,
                  "copy passes align with the 16-row swizzle period");
    auto krow_off = [&](int q) {
        const int r = q / ROW_CH;
        return (uint32_t)r * (uint32_t)K * (uint32_t)EB + (uint32_t)(((q % ROW_CH) ^ swz_krow<ROW_CH>(r)) * 16);
    };
    const uint32_t a_off = krow_off(tid);
    uint32_t b_off[NPAT];
#pragma unroll
    for (int i = 0; i < NPAT; ++i) {
        const int q = i * C::NTHREADS + tid;
        if constexpr (C::TRANS_B) {
            b_off[i] = krow_off(q);
        } else {
            const int k = q / NROW_CH;
            b_off[i] = (uint32_t)k * (uint32_t)N * (uint32_t)EB +
                       (uint32_t)(((q % NROW_CH) ^ swz_nrow<NROW_CH, In::TRK, MB>(k)) * 16);
        }
    }
    const uint32_t smem_addr = lds_addr(smem);
    // the tile's origin inside the matrix and the first row / column it owns
    // (workgroup-uniform: kept in scalar registers, which the vector register
    // file, full with accumulators and fragments, cannot spare)
    auto origin = [&](int t, int& m0, int& n0, int& m_own, int& n_own) {
        int tm, tn;
        tile_coords(t, args.tiles_m, args.tiles_n, args.panel, args.nxcd, tm, tn);
        m_own = __builtin_amdgcn_readfirstlane(tm * BM);
        n_own = __builtin_amdgcn_readfirstlane(tn * BN);
        m0 = __builtin_amdgcn_readfirstlane(min(m_own, M - BM));
        n0 = __builtin_amdgcn_readfirstlane(min(n_own, N - BN));
    };
    auto a_base = [&](int m0) { return args.A + (size_t)m0 * (size_t)K * EB; };
    auto b_base = [&](int n0) {
        return C::TRANS_B ? args.B + (size_t)n0 * (size_t)K * EB : args.B + (size_t)n0 * EB;
    };
    // copy r (< LOADS) of K step u of the tile whose operands start at ga0, gb0,
    // into ring stage st
    auto copy_one = [&](const unsigned char* ga0, const unsigned char* gb0, int u, int st, int r) {
        const uint32_t sa = smem_addr + st * C::STAGE_BYTES;
        if (r < APT) {
            dma16(ga0 + (size_t)u * BK * EB + (size_t)(r * RPP) * K * EB, a_off,
                  sa + (r * C::NWAVES + wave) * 1024);
        } else {
            const int i = r - APT;
            const unsigned char* gb =
                C::TRANS_B ? gb0 + (size_t)u * BK * EB + (size_t)(i * RPP) * K * EB
                           : gb0 + ((size_t)u * BK + (size_t)((i - i % NPAT) * KPP)) * (size_t)N * EB;
            dma16(gb, b_off[i % NPAT], sa + C::A_BYTES + (i * C::NWAVES + wave) * 1024);
        }
    };

    // ---- fragment reads (per lane, relative to a stage's A / B region)
    const int wave_m = wave / C::WAVES_N, wave_n = wave % C::WAVES_N;
    const int wm0 = wave_m * C::WM, wn0 = wave_n * C::WN;
    const int lr = lane % MB, g = lane / MB;
    uint32_t a_rd[FRAG_CH];
#pragma unroll
    for (int x = 0; x < FRAG_CH; ++x) {
        const int r = wm0 + lr;
        a_rd[x] = (uint32_t)(r * BK * EB + (((g * FRAG_CH + x) ^ swz_krow<ROW_CH>(r)) * 16));
    }
    constexpr int B_RD_T = C::TRANS_B ? FRAG_CH : TR_READS;
    uint32_t b_rd[C::TRANS_B ? 1 : TN][B_RD_T];
    if constexpr (C::TRANS_B) {
#pragma unroll
        for (int x = 0; x < FRAG_CH; ++x) {
            const int r = wn0 + lr;
            b_rd[0][x] = (uint32_t)(r * BK * EB + (((g * FRAG_CH + x) ^ swz_krow<ROW_CH>(r)) * 16));
        }
    } else {
        // transpose reads: 16-lane group h = k group; lane i16 supplies k row
        // 8 h + i16 / LPR (+ TRK t) and the 8 bytes of columns (i16 % LPR) 4 ..
        constexpr int TRK = In::TRK, LPR = 16 / TRK;
        const int h = lane >> 4, i16 = lane & 15;
        const int kk = (In::KMF / NG) * h + i16 / LPR;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int t = 0; t < B_RD_T; ++t) {
                const int n = wn0 + MB * j + (i16 % LPR) * (8 / EB);
                const int k = kk + t * TRK;
                const int phys = ((n * EB) >> 4) ^ swz_nrow<NROW_CH, TRK, MB>(k);
                b_rd[j][t] = (uint32_t)(k * BN * EB + phys * 16 + ((n * EB) & 15));
            }
    }
    struct Frags {
        Op a[TM], b[TN];
    };
    Frags fr;
    constexpr int QA = TM * FRAG_CH;
    constexpr int QB = C::TRANS_B ? FRAG_CH : TR_READS;     // reads per B block
    // read op q of the step held in ring stage st: A block q / FRAG_CH, then
    // B block (q - QA) / QB
    auto read_op = [&](int st, int q) {
        const GR_LDS unsigned char* sa = smem + st * C::STAGE_BYTES;
        const GR_LDS unsigned char* sb = sa + C::A_BYTES;
        if (q < QA) {
            const int i = q / FRAG_CH, x = q % FRAG_CH;
            const u32x4_t v = lds_read_b128(sa + a_rd[x] + i * MB * BK * EB);
            if (x == 0)
                In::template set_chunk<0>(fr.a[i], v);
            else
                In::template set_chunk<1>(fr.a[i], v);
        } else if constexpr (C::TRANS_B) {
            const int j = (q - QA) / FRAG_CH, x = (q - QA) % FRAG_CH;
            const u32x4_t v = lds_read_b128(sb + b_rd[0][x] + j * MB * BK * EB);
            if (x == 0)
                In::template set_chunk<0>(fr.b[j], v);
            else
                In::template set_chunk<1>(fr.b[j], v);
        } else {
            const int j = (q - QA) / TR_READS, t = (q - QA) % TR_READS;
            In::set_tr(fr.b[j], t, sb + b_rd[j][t]);
        }
    };

    Acc acc[TM][TN];
    auto clear_acc = [&] {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < In::NACC; ++r) acc[i][j][r] = 0.0f;
    };

    // One K step: the MFMAs of the fragments in fr, with COPIES copies (of K
    // step u of the tile at ga0, gb0, into stage ld_st) and, with READS, each
    // fragment reloaded in place from stage rd_st after its last use (eight
    // regions: A rows in pairs against B blocks 0 .. TN/2-1, then against the
    // rest; B blocks after each half, A rows after their region of the second).
    constexpr int HB = TN / 2;
    auto step = [&](const unsigned char* ga0, const unsigned char* gb0, int u, int ld_st, int rd_st) {
        static_for<0, 8>([&](auto r_tag) {
            constexpr int r = decltype(r_tag)::value;
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (r < LOADS) copy_one(ga0, gb0, u, ld_st, r);
            constexpr int half = r / 4, i0 = 2 * (r % 4);
#pragma unroll
            for (int di = 0; di < 2; ++di)
#pragma unroll
                for (int jj = 0; jj < HB; ++jj) {
                    const int i = i0 + di;
                    const int j = HB * half + (di ? HB - 1 - jj : jj);
                    acc[i][j] = In::mfma(fr.b[j], fr.a[i], acc[i][j]);
                }
            if constexpr (r == 3 || r == 7) {
#pragma unroll
                for (int q = QA + HB * half * QB; q < QA + (HB * half + HB) * QB; ++q) read_op(rd_st, q);
            }
            if constexpr (r >= 4) {
#pragma unroll
                for (int q = i0 * FRAG_CH; q < (i0 + 2) * FRAG_CH; ++q) read_op(rd_st, q);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    // Wait at the top of a step: this wave's copies of the next step have
    // landed (one step's LOADS copies were issued after them; any C stores
    // issued since are waited for as well), then every wave's have, and every
    // wave is past its reads of the stage this step's copies refill (those
    // reads fed the MFMAs of the step before).
    auto top = [&] {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(LOADS));
        asm volatile("s_barrier" ::: "memory");
    };

    // ---- epilogue: ReLU, convert, store from the accumulators.  Lane owns
    // C[m][n .. n+3], m = m0 + wm0 + 16 i + lr, n = n0 + wn0 + 16 j + 4 g.
    constexpr int OB = OutTraits<C::OUT_DT>::bytes;
    auto store_tile = [&](int m0, int n0, int m_own, int n_own) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int m = m0 + wm0 + MB * i + lr;
            if (m < m_own) continue;
            unsigned char* crow = args.C + (size_t)m * (size_t)N * OB;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n = n0 + wn0 + MB * j + 4 * g;
                if (n + 4 <= n_own) continue;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = relu(acc[i][j][e]);
                if constexpr (C::OUT_DT == DT_F32) {
                    float* dst = reinterpret_cast<float*>(crow) + n;
                    if (n >= n_own) {
                        const u32x4_t w = {__builtin_bit_cast(unsigned, v[0]), __builtin_bit_cast(unsigned, v[1]),
                                           __builtin_bit_cast(unsigned, v[2]), __builtin_bit_cast(unsigned, v[3])};
                        __builtin_memcpy(dst, &w, 16);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e >= n_own) dst[e] = v[e];
                    }
                } else {
                    unsigned short hv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) hv[e] = OutTraits<C::OUT_DT>::cvt(v[e]);
                    unsigned short* dst = reinterpret_cast<unsigned short*>(crow) + n;
                    if (n >= n_own) {
                        const u32x2_t w = {hv[0] | ((unsigned)hv[1] << 16), hv[2] | ((unsigned)hv[3] << 16)};
                        __builtin_memcpy(dst, &w, 8);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e >= n_own) dst[e] = hv[e];
                    }
                }
            }
        }
    };

    // ---- the stream: prologue of the first tile
    int m0, n0, m_own, n_own;
    origin(tile, m0, n0, m_own, n_own);
    const unsigned char* ga0 = a_base(m0);
    const unsigned char* gb0 = b_base(n0);
#pragma unroll
    for (int st = 0; st < S - 1; ++st)
#pragma unroll
        for (int r = 0; r < LOADS; ++r) copy_one(ga0, gb0, st, st, r);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((S - 2) * LOADS));
    asm volatile("s_barrier" ::: "memory");
#pragma unroll
    for (int q = 0; q < C::NR; ++q) read_op(0, q);

    uint32_t gbase = 0;     // stream position of the tile's first K step
    for (;;) {
        const int next = tile + G;
        const bool has_next = next < total;
        // After the workgroup's last tile the stream runs on into a copy of
        // that tile's first steps, which nobody reads: one schedule for every
        // tile (a separate ending made the register allocator spill).
        int m1 = m0, n1 = n0, m1_own = m_own, n1_own = n_own;
        if (has_next) origin(next, m1, n1, m1_own, n1_own);
        const unsigned char* ga1 = a_base(m1);
        const unsigned char* gb1 = b_base(n1);
        clear_acc();
        // steps whose copies fetch this tile's own steps
        int t = 0;
        for (; t < nk - (S - 1); ++t) {
            top();
            step(ga0, gb0, t + S - 1, (gbase + t + S - 1) % S, (gbase + t + 1) % S);
        }
        // the last S-1 steps fetch the next tile's first S-1 steps, and the
        // last one reloads the fragments of the next tile's first step
        for (; t < nk; ++t) {
            top();
            step(ga1, gb1, t + S - 1 - nk, (gbase + t + S - 1) % S, (gbase + t + 1) % S);
        }
        store_tile(m0, n0, m_own, n_own);
        if (!has_next) {
            // no copy may still be writing LDS when the workgroup retires
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            break;
        }
        tile = next;
        m0 = m1;
        n0 = n1;
        m_own = m1_own;
        n_own = n1_own;
        ga0 = ga1;
        gb0 = gb1;
        gbase += nk;
    }
}

// One workgroup per tile, or (persistent configurations, the T.Persistent form
// of page "TileLang：GPU/NPU 通用算子 DSL", §3.3) a grid of at most one
// workgroup per CU whose workgroups walk the tiles wg, wg + grid, ...: the
// accumulator is cleared per tile, and a barrier after each tile keeps the
// next tile's copies off the LDS the epilogue may still be reading.  A grid
// that is a multiple of 8 keeps every tile of a workgroup on its XCD.
//
// Stream-K configurations (the published Stream-K decomposition, Osama et al.,
// 2023, in its data-parallel + stream-K hybrid): the first dp_tiles workgroups
// take whole tiles; the remaining tiles' K steps, ceil(K / BK) per tile, are
// laid end to end and split into sk_units near-equal ranges, one per further
// workgroup.  A range crosses at most a few tile boundaries; each part of it in
// one tile is a piece.  Pieces never wait for one another: each publishes its
// partial and counts itself in at the tile's counter, and the last to arrive
// finishes the tile, so no workgroup depends on another being resident.
template <class C>
__global__ void __launch_bounds__(C::NTHREADS, 1) gemm_relu_kernel(KernelArgs args)
{
    __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[C::LDS_BYTES];
    GR_LDS unsigned char* smem = (GR_LDS unsigned char*)(smem_raw);
    if constexpr (C::STREAMK) {
        __shared__ SkState sk_raw;
        GR_LDS SkState* sk = (GR_LDS SkState*)(&sk_raw);
        const int iters = (args.K + C::BK - 1) / C::BK;
        const int u = (int)blockIdx.x - args.dp_tiles;
        // unit w takes steps [lo(w), lo(w + 1)) of the split tiles' sequence;
        // a whole-tile workgroup (u < 0) runs the loop once over its tile
        auto split = [&](int& q, int& r) {
            const int total = (args.tiles_m * args.tiles_n - args.dp_tiles) * iters;
            q = total / args.sk_units;
            r = total % args.sk_units;
        };
        if (threadIdx.x == 0) {
            int q, r;
            split(q, r);
            sk->lo = u < 0 ? 0 : u * q + min(u, r);
            sk->hi = u < 0 ? iters : (u + 1) * q + min(u + 1, r);
        }
        for (;;) {
            barrier_lds();      // the state is written; the last tile's epilogue is done with LDS
            const int lo = sk->lo, hi = sk->hi;
            if (lo >= hi) break;
            barrier_lds();      // every wave has read lo before thread 0 advances it
            if (threadIdx.x == 0) {
                SkPiece pc;
                if (u < 0) {
                    pc = SkPiece{0, iters, 0, 1, 0, 0, 0};
                    sk->wg = blockIdx.x;
                } else {
                    int q, r;
                    split(q, r);
                    auto lo_of = [&](int w) { return w * q + min(w, r); };
                    auto unit_of = [&](int x) {
                        return x < r * (q + 1) ? x / (q + 1) : r + (x - r * (q + 1)) / q;
                    };
                    const int t = lo / iters, t0 = t * iters;
                    pc.kt0 = lo - t0;
                    pc.kt1 = min(iters, pc.kt0 + hi - lo);
                    pc.tile = t;
                    pc.first = unit_of(t0);
                    pc.count = unit_of(t0 + iters - 1) - pc.first + 1;
                    pc.pos = u - pc.first;
                    pc.slot0 = 2 * pc.first + (lo_of(pc.first) < t0 ? 1 : 0);
                    sk->wg = args.dp_tiles + t;
                }
                // field by field: no assignment operator into an LDS object
                sk->pc.kt0 = pc.kt0;
                sk->pc.kt1 = pc.kt1;
                sk->pc.tile = pc.tile;
                sk->pc.count = pc.count;
                sk->pc.pos = pc.pos;
                sk->pc.first = pc.first;
                sk->pc.slot0 = pc.slot0;
                sk->lo = lo + pc.kt1 - pc.kt0;
            }
            barrier_lds();
            gemm_relu_tile<C>(args, sk->wg, smem, sk, Region{args.tiles_m, args.tiles_n, args.panel, 0});
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        }
    } else if constexpr (C::PERSISTENT && C::MB == 16) {
        gemm_relu_i16_persistent<C>(args, smem);
    } else if constexpr (C::PERSISTENT) {
        const int total = args.tiles_m * args.tiles_n;
        for (int wg = blockIdx.x; wg < total; wg += gridDim.x) {
            gemm_relu_tile<C>(args, wg, smem, nullptr, Region{args.tiles_m, args.tiles_n, args.panel, 0});
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            barrier_lds();
        }
    } else if constexpr (C::SPLITK) {
        gemm_relu_tile<C>(args, (int)blockIdx.x % (args.tiles_m * args.tiles_n), smem, nullptr,
                          Region{args.tiles_m, args.tiles_n, args.panel, 0});
    } else {
        gemm_relu_tile<C>(args, blockIdx.x, smem, nullptr,
                          Region{args.tiles_m, args.tiles_n, args.panel, 0});
    }
}

// Whole-tile rounds with a narrower last round: the first tiles1 workgroups
// (whole rounds of CUs) take C1 tiles over the columns [0, n_org2), the rest
// take C2 tiles over [n_org2, N) — one round of narrower tiles instead of a
// partly idle round of full ones.  No tile depends on another, so the two
// kinds need no synchronisation; the dispatcher starts a C2 workgroup on each
// CU as its last C1 workgroup retires.  This is the scheduling aim of the
// T.Persistent form of page "TileLang：GPU/NPU 通用算子 DSL", §3.3 (every CU
// busy to the end), reached with whole tiles instead of a tile loop.
template <class C1, class C2>
__global__ void __launch_bounds__(C1::NTHREADS, 1) gemm_relu_kernel_2r(KernelArgs args)
{
    static_assert(C1::NTHREADS == C2::NTHREADS && !C1::STREAMK && !C2::STREAMK &&
                      !C1::PERSISTENT && !C2::PERSISTENT,
                  "two-region grids: whole tiles of two configurations with one block size");
    constexpr int LDS = C1::LDS_BYTES > C2::LDS_BYTES ? C1::LDS_BYTES : C2::LDS_BYTES;
    __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[LDS];
    GR_LDS unsigned char* smem = (GR_LDS unsigned char*)(smem_raw);
    const int wg = blockIdx.x;
    if (wg < args.tiles1)
        gemm_relu_tile<C1>(args, wg, smem, nullptr, Region{args.tiles_m, args.tiles_n, args.panel, 0});
    else
        gemm_relu_tile<C2>(args, wg - args.tiles1, smem, nullptr,
                           Region{args.tiles_m2, args.tiles_n2, args.panel2, args.n_org2});
}

}  // namespace gemm_relu_hip
