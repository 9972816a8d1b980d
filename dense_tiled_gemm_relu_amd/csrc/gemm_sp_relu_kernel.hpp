// 2:4 structured-sparse GEMM + ReLU for CDNA4 (gfx950): C = max(A·op(B), 0)
// with A given compressed.
//
// The operation is the T.gemm_sp item of page "TileLang：GPU/NPU 通用算子 DSL"
// (§4.1 timeline: 2:4 structured-sparse tensor-core GEMM); page "从 TVM 到
// TileLang…", §四, describes its shape: the compressed A and its metadata E
// are brought in side by side, already arranged before they reach shared
// memory, and the tile gemm consumes both.  The pages fix no format; this
// library reads it as follows (the oracle decodes the same one):
//   * every row of A is cut along K into groups of 4 with at most two
//     non-zeros; As (M, K/2) keeps the two stored values of group q at
//     As[i][2q], As[i][2q+1];
//   * E gives their positions p0 < p1 inside the group as the nibble
//     p0 | p1 << 2; E is blocked by 64 columns of K — block kb holds 8 bytes
//     per row (M x 8), group q of row i in nibble q % 2 (low first) of byte
//     (q % 16) / 2 of that row's 8 bytes — so one K step of 64 finds the
//     metadata of a tile's rows in one contiguous run.
//
// On gfx950 the contraction is v_smfmac_f32_32x32x32_{f16,bf16} (the sparse
// operand is the instruction's first source, so a lane owns 4 consecutive
// rows m of one column n of the 32x32 C block).  Its lane layout, checked on
// the device by probe_smfmac_raw: lane 32 g + i of the sparse operand holds
// the 8 stored values of groups 4 g .. 4 g + 3 of the 32-wide k step of row i
// (one 16-byte chunk of the compressed row) and, in bits 0..15 of its index
// word, their 4 nibbles in group order — two consecutive bytes of E; lane
// 32 g + j of the dense operand holds k = 8 g .. 8 g + 7 and 16 + 8 g ..
// 16 + 8 g + 7 of column j (two 16-bit dense k steps back to back).
//
// Pipeline: the direct global -> LDS copies of the dense kernel (A, B and the
// metadata of a 64-wide K step per stage, in an S-stage ring), two sparse
// k steps per stage, fragments of the next k step read while the current one
// is contracted, and a register-staged, zero-filled step for a K tail.
#pragma once

#include "gemm_relu_kernel.hpp"

namespace gemm_relu_hip {

struct SpArgs {
    const unsigned char* As;  // (M, K/2) compressed A, 16-bit elements
    const unsigned char* E;   // ceil(K/64) blocks of (M, 8) metadata bytes
    const unsigned char* B;   // (K, N) row-major, or (N, K) when transposed
    unsigned char* C;         // (M, N) row-major, 2- or 4-byte elements
    int M, N, K;
    int tiles_m, tiles_n;
    int panel;
    int nxcd;
};

typedef _Float16 f16x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x16_t __attribute__((ext_vector_type(16)));

// Direct global -> LDS copy of 4 bytes per lane (global_load_lds_dword):
// lane i's bytes land at LDS address M0 + 4 i; tracked with vmcnt like dma16.
__device__ __forceinline__ void dma4(const unsigned char* gbase, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "s_nop 0\n\t"
                 "global_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(gbase), "s"(lds)
                 : "memory", "m0");
}

template <int IN_DT_, int OUT_DT_, bool TRANS_B_, int STAGES_ = 3, int WAVES_N_ = 2> struct SpCfg {
    static constexpr int IN_DT = IN_DT_, OUT_DT = OUT_DT_;
    static constexpr bool TRANS_B = TRANS_B_;
    static constexpr int BM = 256, BN = 256, BK = 64;           // BK in K (2 sparse k steps)
    // 2 x 2 waves of 128 x 128, or 2 x 4 of 128 x 64 (two waves per SIMD)
    static constexpr int WAVES_M = 2, WAVES_N = WAVES_N_, NWAVES = WAVES_M * WAVES_N, NTHREADS = 64 * NWAVES;
    static constexpr int STAGES = STAGES_;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, TM = WM / 32, TN = WN / 32;
    static constexpr int KSUB = BK / 32;
    // per stage: compressed A rows of BK/2 values (64 bytes, 4 chunks), B
    // (N,K) rows of BK values (8 chunks) or (K,N) rows of BN values (32
    // chunks), and the metadata of BM rows (8 bytes each)
    static constexpr int A_ROW_CH = BK / 2 * 2 / 16;
    static constexpr int B_ROW_CH = BK * 2 / 16;
    static constexpr int NROW_CH = BN * 2 / 16;
    static constexpr int A_BYTES = BM * BK;
    static constexpr int B_BYTES = BN * BK * 2;
    static constexpr int E_BYTES = BM * 8;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + E_BYTES;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static constexpr int APT = A_BYTES / 16 / NTHREADS;         // 16-byte copies per thread
    static constexpr int BPT = B_BYTES / 16 / NTHREADS;
    static constexpr int EPT = E_BYTES / 4 / NTHREADS;          // 4-byte copies per thread
    static constexpr int LOADS_PER_STAGE = APT + BPT + EPT;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity of a gfx950 CU");
    static_assert((STAGES - 2) * LOADS_PER_STAGE < 64, "vmcnt range");
    static_assert(APT * NTHREADS * 16 == A_BYTES && BPT * NTHREADS * 16 == B_BYTES &&
                      EPT * NTHREADS * 4 == E_BYTES,
                  "loader tiling");
};

template <int IN_DT> struct SpIn;
// Operands travel as dword vectors (4 for the sparse one, 8 for the dense
// one), filled in place part by part.
typedef int i32x4s_t __attribute__((ext_vector_type(4)));
template <> struct SpIn<DT_F16> {
    __device__ static f32x16_t smfmac(i32x4s_t a, i32x8_t b, f32x16_t c, int idx)
    {
        return __builtin_amdgcn_smfmac_f32_32x32x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                        __builtin_bit_cast(f16x16_t, b), c, idx,
                                                        0, 0);
    }
};
template <> struct SpIn<DT_BF16> {
    __device__ static f32x16_t smfmac(i32x4s_t a, i32x8_t b, f32x16_t c, int idx)
    {
        return __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                         __builtin_bit_cast(bf16x16_t, b), c, idx,
                                                         0, 0);
    }
};

template <class C>
__global__ void __launch_bounds__(C::NTHREADS, 1) gemm_sp_relu_kernel(SpArgs args)
{
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, S = C::STAGES;
    constexpr int TM = C::TM, TN = C::TN, KSUB = C::KSUB;
    constexpr int APT = C::APT, BPT = C::BPT, EPT = C::EPT;
    constexpr int A_ROW_CH = C::A_ROW_CH, B_ROW_CH = C::B_ROW_CH, NROW_CH = C::NROW_CH;

    __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[C::LDS_BYTES];
    GR_LDS unsigned char* smem = (GR_LDS unsigned char*)(smem_raw);
    const uint32_t smem_addr = lds_addr(smem);

    const int M = args.M, N = args.N, K = args.K;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int KH = K / 2;                                        // compressed row length

    int tm, tn;
    tile_coords(blockIdx.x, args.tiles_m, args.tiles_n, args.panel, args.nxcd, tm, tn);
    const int m0 = tm * BM;
    // (K,N) B: the last tile column moves back to end at N (needs N >= BN);
    // its shared columns are recomputed identically and stored twice
    const int n0 = C::TRANS_B ? tn * BN : min(tn * BN, N - BN);
    const int nk = K / BK;                                       // full steps

    // ---- loader geometry (slot q = i NTHREADS + tid of a stage region)
    uint32_t a_src[APT];
#pragma unroll
    for (int i = 0; i < APT; ++i) {
        const int q = i * C::NTHREADS + tid;
        const int r = q / A_ROW_CH, c = (q % A_ROW_CH) ^ swz_krow<A_ROW_CH>(r);
        const int row = min(m0 + r, M - 1) - m0;
        a_src[i] = (uint32_t)row * (uint32_t)KH * 2u + (uint32_t)c * 16u;
    }
    uint32_t b_src[BPT];
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        const int q = i * C::NTHREADS + tid;
        if constexpr (C::TRANS_B) {
            const int r = q / B_ROW_CH, c = (q % B_ROW_CH) ^ swz_krow<B_ROW_CH>(r);
            const int row = min(n0 + r, N - 1) - n0;
            b_src[i] = (uint32_t)row * (uint32_t)K * 2u + (uint32_t)c * 16u;
        } else {
            const int k = q / NROW_CH, c = (q % NROW_CH) ^ swz_nrow<NROW_CH, 4, 32>(k);
            b_src[i] = (uint32_t)k * (uint32_t)N * 2u + (uint32_t)c * 16u;
        }
    }
    // metadata: 4-byte piece q of a stage's (BM x 8)-byte block, rows clamped
    uint32_t e_src[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int q = i * C::NTHREADS + tid;
        const int row = min(m0 + q / 2, M - 1) - m0;
        e_src[i] = (uint32_t)row * 8u + (uint32_t)(q % 2) * 4u;
    }
    const unsigned char* a_tile = args.As + (size_t)m0 * (size_t)KH * 2;
    const unsigned char* b_tile = C::TRANS_B ? args.B + (size_t)n0 * (size_t)K * 2 : args.B + (size_t)n0 * 2;

    auto issue_stage = [&](int t, int stage) {
        const uint32_t sa = smem_addr + stage * C::STAGE_BYTES;
        const uint32_t sb = sa + C::A_BYTES;
        const uint32_t se = sb + C::B_BYTES;
        const unsigned char* ga = a_tile + (size_t)t * (BK / 2) * 2;
        const unsigned char* gb = C::TRANS_B ? b_tile + (size_t)t * BK * 2
                                             : b_tile + (size_t)t * BK * (size_t)N * 2;
        const unsigned char* ge = args.E + ((size_t)t * (size_t)M + (size_t)m0) * 8;
#pragma unroll
        for (int i = 0; i < APT; ++i) dma16(ga, a_src[i], sa + (i * C::NWAVES + wave) * 1024);
#pragma unroll
        for (int i = 0; i < BPT; ++i) dma16(gb, b_src[i], sb + (i * C::NWAVES + wave) * 1024);
#pragma unroll
        for (int i = 0; i < EPT; ++i) dma4(ge, e_src[i], se + (i * C::NWAVES + wave) * 256);
    };
    // copy l (< LOADS_PER_STAGE: A chunks, B chunks, metadata pieces) of stage t
    auto issue_one = [&](int t, int stage, int l) {
        const uint32_t sa = smem_addr + stage * C::STAGE_BYTES;
        const uint32_t sb = sa + C::A_BYTES;
        const uint32_t se = sb + C::B_BYTES;
        if (l < APT) {
            dma16(a_tile + (size_t)t * (BK / 2) * 2, a_src[l], sa + (l * C::NWAVES + wave) * 1024);
        } else if (l < APT + BPT) {
            const unsigned char* gb = C::TRANS_B ? b_tile + (size_t)t * BK * 2
                                                 : b_tile + (size_t)t * BK * (size_t)N * 2;
            dma16(gb, b_src[l - APT], sb + ((l - APT) * C::NWAVES + wave) * 1024);
        } else {
            const unsigned char* ge = args.E + ((size_t)t * (size_t)M + (size_t)m0) * 8;
            dma4(ge, e_src[l - APT - BPT], se + ((l - APT - BPT) * C::NWAVES + wave) * 256);
        }
    };

    // ---- K tail (K % 64): one register-staged step, zero-filled past K; the
    // metadata block of the tail exists whole, so it takes the direct copy.
    auto fill_tail = [&](int stage) {
        GR_LDS unsigned char* sa = smem + stage * C::STAGE_BYTES;
        GR_LDS unsigned char* sb = sa + C::A_BYTES;
        const int t = nk;
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int q = i * C::NTHREADS + tid;
            const int r = q / A_ROW_CH, c = (q % A_ROW_CH) ^ swz_krow<A_ROW_CH>(r);
            const int e0 = t * (BK / 2) + 8 * c;                 // compressed element
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (m0 + r < M) {
                const unsigned short* p =
                    reinterpret_cast<const unsigned short*>(args.As) + (size_t)(m0 + r) * KH + e0;
                unsigned short h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) h[e] = (e0 + e < KH) ? p[e] : (unsigned short)0;
                v = u32x4_t{h[0] | ((unsigned)h[1] << 16), h[2] | ((unsigned)h[3] << 16),
                            h[4] | ((unsigned)h[5] << 16), h[6] | ((unsigned)h[7] << 16)};
            }
            *reinterpret_cast<GR_LDS u32x4_t*>(sa + q * 16) = v;
        }
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            const int q = i * C::NTHREADS + tid;
            unsigned short h[8];
            if constexpr (C::TRANS_B) {
                const int r = q / B_ROW_CH, c = (q % B_ROW_CH) ^ swz_krow<B_ROW_CH>(r);
                const int k0 = t * BK + 8 * c;
                const bool ok = n0 + r < N;
                const unsigned short* p =
                    reinterpret_cast<const unsigned short*>(args.B) + (size_t)(n0 + r) * K + k0;
#pragma unroll
                for (int e = 0; e < 8; ++e) h[e] = (ok && k0 + e < K) ? p[e] : (unsigned short)0;
            } else {
                const int k = q / NROW_CH, c = (q % NROW_CH) ^ swz_nrow<NROW_CH, 4, 32>(k);
                const int kk = t * BK + k;
                const unsigned short* p =
                    reinterpret_cast<const unsigned short*>(args.B) + (size_t)kk * N + n0 + 8 * c;
#pragma unroll
                for (int e = 0; e < 8; ++e) h[e] = (kk < K) ? p[e] : (unsigned short)0;
            }
            *reinterpret_cast<GR_LDS u32x4_t*>(sb + q * 16) =
                u32x4_t{h[0] | ((unsigned)h[1] << 16), h[2] | ((unsigned)h[3] << 16),
                        h[4] | ((unsigned)h[5] << 16), h[6] | ((unsigned)h[7] << 16)};
        }
        const uint32_t se = smem_addr + stage * C::STAGE_BYTES + C::A_BYTES + C::B_BYTES;
        const unsigned char* ge = args.E + ((size_t)t * (size_t)M + (size_t)m0) * 8;
#pragma unroll
        for (int i = 0; i < EPT; ++i) dma4(ge, e_src[i], se + (i * C::NWAVES + wave) * 256);
    };

    // ---- fragment read geometry
    const int wave_m = wave / C::WAVES_N, wave_n = wave % C::WAVES_N;
    const int wm0 = wave_m * C::WM, wn0 = wave_n * C::WN;
    const int lr = lane & 31, g = lane >> 5;
    // compressed A row wm0 + 32 i + lr, chunk 2 s + g
    uint32_t a_rd[KSUB];
#pragma unroll
    for (int s = 0; s < KSUB; ++s) {
        const int r = wm0 + lr;
        a_rd[s] = (uint32_t)(r * A_ROW_CH * 16 + (((2 * s + g) ^ swz_krow<A_ROW_CH>(r)) * 16));
    }
    // B: (N,K) rows, chunks 4 s + g and 4 s + 2 + g; (K,N): 4 transpose reads
    // of 4 k rows: k = 32 s + 16 (t / 2) + 8 g' + 4 (t % 2) + i16 / 4 for the
    // 16-lane group h = 2 g' + nh, column 16 nh + 4 (i16 % 4) of the block
    uint32_t b_rd[C::TRANS_B ? KSUB : TN][2];
    if constexpr (C::TRANS_B) {
#pragma unroll
        for (int s = 0; s < KSUB; ++s)
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int r = wn0 + lr;
                b_rd[s][x] = (uint32_t)(r * B_ROW_CH * 16 +
                                        (((4 * s + 2 * x + g) ^ swz_krow<B_ROW_CH>(r)) * 16));
            }
    } else {
        const int h = lane >> 4, i16 = lane & 15;
        const int gk = h >> 1, nh = h & 1;
        const int kk = 8 * gk + i16 / 4;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = wn0 + 32 * j + 16 * nh + (i16 % 4) * 4;
            const int phys = ((n * 2) >> 4) ^ swz_nrow<NROW_CH, 4, 32>(kk);
            b_rd[j][0] = (uint32_t)(kk * BN * 2 + phys * 16 + ((n * 2) & 15));
            b_rd[j][1] = 0;
        }
    }
    // metadata: row wm0 + 32 i + lr, bytes 4 s + 2 g, +1
    const uint32_t e_rd = (uint32_t)((wm0 + lr) * 8 + 2 * g);

    // Fragments: A and the index words double-buffered (the next k step's
    // are read while the current one is contracted); B single-buffered —
    // block j of the next k step is read into b[j] right after the current
    // k step's last use of it (MFMAs go block column by block column).
    struct AFrags {
        i32x4s_t a[TM];
        int idx[TM];
    };
    i32x8_t b[TN];
    auto read_a = [&](int stage, int s, AFrags& f) {
        const GR_LDS unsigned char* sa = smem + stage * C::STAGE_BYTES;
        const GR_LDS unsigned char* se = sa + C::A_BYTES + C::B_BYTES;
#pragma unroll
        for (int i = 0; i < TM; ++i)
            f.a[i] = __builtin_bit_cast(i32x4s_t, lds_read_b128(sa + a_rd[s] + i * 32 * A_ROW_CH * 16));
#pragma unroll
        for (int i = 0; i < TM; ++i)
            f.idx[i] = *reinterpret_cast<const GR_LDS unsigned short*>(se + e_rd + 4 * s + i * 32 * 8);
    };
    auto read_b = [&](int stage, int s, int j) {
        const GR_LDS unsigned char* sb = smem + stage * C::STAGE_BYTES + C::A_BYTES;
        if constexpr (C::TRANS_B) {
            b[j].lo = __builtin_bit_cast(i32x4s_t, lds_read_b128(sb + b_rd[s][0] + j * 32 * B_ROW_CH * 16));
            b[j].hi = __builtin_bit_cast(i32x4s_t, lds_read_b128(sb + b_rd[s][1] + j * 32 * B_ROW_CH * 16));
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const i32x2_t r = __builtin_bit_cast(
                    i32x2_t,
                    lds_read_tr16(sb + b_rd[j][0] + (32 * s + 16 * (t / 2) + 4 * (t % 2)) * BN * 2));
                b[j][2 * t] = r[0];
                b[j][2 * t + 1] = r[1];
            }
        }
    };

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    // contract with A set f; if next_stage >= 0, refill b[] with k step
    // next_s of next_stage as the blocks retire
    auto contract = [&](const AFrags& f, int next_stage, int next_s) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            // A blocks in snake order (down the column for odd j), so the
            // compressed operand is unchanged where j steps
#pragma unroll
            for (int ii = 0; ii < TM; ++ii) {
                const int i = (j & 1) ? TM - 1 - ii : ii;
                acc[i][j] = SpIn<C::IN_DT>::smfmac(f.a[i], b[j], acc[i][j], f.idx[i]);
            }
            if (next_stage >= 0) read_b(next_stage, next_s, j);
        }
    };

    // ---- pipeline: S-1 stages in flight ahead of the one contracted.  The
    // copies of stage t+S-1 are spread over step t: each k step is TN
    // scheduling regions (block column j: its copies, its MFMAs, then the
    // read of its next B block), with LK copies per k step.  At the last k
    // step of stage t the wave waits for stage t+1 (the copies issued after
    // it: stages t+2 .. t+S-2 whole and the first k steps' share of stage
    // t+S-1), meets the others at a barrier (which also retires every read of
    // stage t, so its buffer may be refilled) and reads stage t+1's first
    // fragments.
    constexpr int L = C::LOADS_PER_STAGE, LK = (L + KSUB - 1) / KSUB;
    constexpr int ALLOW = (S - 3) * L + (KSUB - 1) * LK;
    static_assert(ALLOW < 64, "vmcnt range");
    AFrags fa[2];
#pragma unroll
    for (int st = 0; st < S - 1; ++st)
        if (st < nk) issue_stage(st, st);
    if (nk > 0) {
        if (nk - 1 >= S - 2)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm((S - 2) * L));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        barrier_lds();
        read_a(0, 0, fa[0]);
#pragma unroll
        for (int j = 0; j < TN; ++j) read_b(0, 0, j);
    }
    // one step; STEADY: the stage S-1 ahead exists (no run-time checks).
    // ring: the step's ring position, t mod S, as a compile-time constant in
    // the unrolled steady loop (so that every LDS address of the step is a
    // per-lane base plus a constant), or at run time
    auto step = [&](int t, auto steady_tag, auto ring) {
        constexpr bool STEADY = decltype(steady_tag)::value;
        const int stage = ring;
        const bool loads = STEADY || t + S - 1 < nk;
        const int ld_stage = stage == 0 ? S - 1 : stage - 1;
#pragma unroll
        for (int s = 0; s < KSUB; ++s) {
            int next_stage = -1, next_s = 0;
            if (s + 1 < KSUB) {
                next_stage = stage;
                next_s = s + 1;
            } else if (STEADY || t + 1 < nk) {
                if (loads)
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm(ALLOW));
                else
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
                barrier_lds();
                next_stage = stage + 1 == S ? 0 : stage + 1;
            }
            const AFrags& f = fa[s & 1];
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                __builtin_amdgcn_sched_barrier(0);
                if (loads) {
#pragma unroll
                    for (int l = s * LK + (j * LK + TN - 1) / TN; l < s * LK + ((j + 1) * LK + TN - 1) / TN; ++l)
                        if (l < L) issue_one(t + S - 1, ld_stage, l);
                }
                if (j == 0 && next_stage >= 0) read_a(next_stage, next_s, fa[(s + 1) & 1]);
#pragma unroll
                for (int ii = 0; ii < TM; ++ii) {
                    const int i = (j & 1) ? TM - 1 - ii : ii;     // snake order, as above
                    acc[i][j] = SpIn<C::IN_DT>::smfmac(f.a[i], b[j], acc[i][j], f.idx[i]);
                }
                if (next_stage >= 0) read_b(next_stage, next_s, j);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    const int t_steady = nk - (S - 1) > 0 ? nk - (S - 1) : 0;
    int t = 0;
    for (; t + S <= t_steady; t += S)
        static_for<0, S>([&](auto r) { step(t + decltype(r)::value, std::integral_constant<bool, true>{}, r); });
    for (; t < t_steady; ++t) step(t, std::integral_constant<bool, true>{}, t % S);
    for (; t < nk; ++t) step(t, std::integral_constant<bool, false>{}, t % S);
    if (K % BK != 0) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        barrier_lds();
        fill_tail(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        barrier_lds();
        read_a(0, 0, fa[0]);
#pragma unroll
        for (int j = 0; j < TN; ++j) read_b(0, 0, j);
#pragma unroll
        for (int s = 0; s < KSUB; ++s) {
            if (s + 1 < KSUB) read_a(0, s + 1, fa[(s + 1) & 1]);
            contract(fa[s & 1], s + 1 < KSUB ? 0 : -1, s + 1);
        }
    }

    // ---- epilogue: lane owns C[m .. m+3][n] of each block, m = m0 + wm0 +
    // 32 i + 8 (r / 4) + 4 g + (r % 4), n = n0 + wn0 + 32 j + lr: for each
    // register, the 32 lanes of a group store 32 consecutive n of one row.
    constexpr int OB = OutTraits<C::OUT_DT>::bytes;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn0 + 32 * j + lr;
        if (n >= N) continue;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm0 + 32 * i + 8 * (r / 4) + 4 * g + (r % 4);
                if (m >= M) continue;
                const float v = relu(acc[i][j][r]);
                if constexpr (OB == 4)
                    reinterpret_cast<float*>(args.C)[(size_t)m * N + n] = v;
                else
                    reinterpret_cast<unsigned short*>(args.C)[(size_t)m * N + n] =
                        OutTraits<C::OUT_DT>::cvt(v);
            }
    }
}

}  // namespace gemm_relu_hip
