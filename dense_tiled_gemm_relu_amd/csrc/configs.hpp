// Kernel configurations of the fused GEMM + ReLU and their launch table.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_relu_kernel.hpp"

namespace gemm_relu_hip {

// Tile shapes.  "d" = direct global->LDS copies (any shape and alignment; a
// (K,N) B needs one full tile of columns); "g" = register-staged copies with
// element-wise bounds checks (any shape).  BK in a name counts 16-bit
// elements: the 8-bit instantiation of a configuration takes 2 BK elements per
// step, so that a step moves the same bytes.
enum ConfigId : int {
    CFG_D256x256x64_S2 = 0,
    CFG_D256x256x32_S4,
    CFG_D256x256x32_S5,
    CFG_D256x256x32_S4_I,
    CFG_D256x256x64_S2_16,
    CFG_D256x256x32_S4_I16,
    CFG_D256x256x32_S4_IP,
    CFG_D256x256x32_S4_ISK,
    CFG_D256x256x32_S4_W8I,
    CFG_D256x256x32_S5_W8I,
    CFG_D256x256x64_S2_W8,
    CFG_D128x128x64_S3,
    CFG_D128x128x64_S2,
    CFG_D256x128x64_S2,
    CFG_D64x64x64_S4,
    CFG_D64x32x128_S4,
    CFG_D32x64x128_S4,
    CFG_G128x128x64,
    CFG_G64x64x64,
    CFG_D256x192x32_S4_I16,
    CFG_D256x256x32_S4_I16P,
    CFG_D64x128x64_S4_SPLITK,
    CFG_D64x256x64_S3_SPLITK,
    CFG_D64x128x128_S3_SPLITK,
    CFG_D64x128x64_S3_SPLITK,
    CFG_D256x256x32_S4_I16W8,
    CFG_D128x384x32_S4_I16W8,
    CFG_D256x256x32_S4_I16W8SK,
    CFG_COUNT
};

struct ConfigInfo {
    const char* name;
    int bm, bn;
    bool direct;
    bool persistent = false;   // grid of min(tiles, CUs) workgroups looping over tiles
    bool streamk = false;      // whole-tile workgroups, then stream-K units (workspace)
    bool splitk = false;       // every tile split along K: fp32 partials in a caller's workspace
    int bk16 = 0;              // K-split configurations: K elements per step (16-bit inputs)
    int per_cu = 1;            // K-split configurations: workgroups resident per CU
};

inline const ConfigInfo& config_info(int id)
{
    static const ConfigInfo table[CFG_COUNT] = {
        {"d256x256x64_s2", 256, 256, true},
        {"d256x256x32_s4", 256, 256, true},
        {"d256x256x32_s5", 256, 256, true},
        {"d256x256x32_s4_i", 256, 256, true},
        {"d256x256x64_s2_16", 256, 256, true},
        {"d256x256x32_s4_i16", 256, 256, true},
        {"d256x256x32_s4_ip", 256, 256, true, true},
        {"d256x256x32_s4_isk", 256, 256, true, false, true},
        {"d256x256x32_s4_w8i", 256, 256, true},
        {"d256x256x32_s5_w8i", 256, 256, true},
        {"d256x256x64_s2_w8", 256, 256, true},
        {"d128x128x64_s3", 128, 128, true},
        {"d128x128x64_s2", 128, 128, true},
        {"d256x128x64_s2", 256, 128, true},
        {"d64x64x64_s4", 64, 64, true},
        {"d64x32x128_s4", 64, 32, true},
        {"d32x64x128_s4", 32, 64, true},
        {"g128x128x64", 128, 128, false},
        {"g64x64x64", 64, 64, false},
        {"d256x192x32_s4_i16", 256, 192, true},
        {"d256x256x32_s4_i16p", 256, 256, true, true},
        {"d64x128x64_s4_splitk", 64, 128, true, false, false, true, 64, 1},
        {"d64x256x64_s3_splitk", 64, 256, true, false, false, true, 64, 1},
        {"d64x128x128_s3_splitk", 64, 128, true, false, false, true, 128, 1},
        {"d64x128x64_s3_splitk", 64, 128, true, false, false, true, 64, 2},
        {"d256x256x32_s4_i16w8", 256, 256, true},
        {"d128x384x32_s4_i16w8", 128, 384, true},
        {"d256x256x32_s4_i16w8sk", 256, 256, true, false, true},
    };
    return table[id];
}

// Comparison configurations: variants measured against the ones plan selection
// uses and never chosen by it (other stage counts and step depths, 8-wave
// tiles, the bunched 16x16-block tile, the persistent tile loops and the
// stream-K split; for block-scaled inputs the two-stage 256-wide tiles).  They
// are compiled only when the library is built with
// GEMM_RELU_COMPARISON_CONFIGS defined; otherwise GEMM_RELU_FORCE_CONFIG
// cannot select them and the library has no path that allocates device memory.
#ifdef GEMM_RELU_COMPARISON_CONFIGS
inline constexpr bool kComparisonBuilt = true;
#else
inline constexpr bool kComparisonBuilt = false;
#endif

inline constexpr bool comparison_config(int id)
{
    return id == CFG_D256x256x64_S2 || id == CFG_D256x256x32_S4 || id == CFG_D256x256x32_S5 ||
           id == CFG_D256x256x64_S2_16 || id == CFG_D256x256x32_S4_IP ||
           id == CFG_D256x256x32_S4_ISK || id == CFG_D256x256x32_S4_W8I ||
           id == CFG_D256x256x32_S5_W8I || id == CFG_D256x256x64_S2_W8 || id == CFG_D256x128x64_S2 ||
           id == CFG_D256x256x32_S4_I16P || id == CFG_D64x256x64_S3_SPLITK ||
           id == CFG_D64x128x128_S3_SPLITK || id == CFG_D64x128x64_S3_SPLITK ||
           id == CFG_D128x384x32_S4_I16W8 || id == CFG_D256x256x32_S4_I16W8SK;
}

// Whether this build of the library holds kernels of configuration id.
inline constexpr bool config_built(int id)
{
    return kComparisonBuilt || !comparison_config(id);
}

// K elements per step of a configuration whose 16-bit step is BK16 elements.
// Block-scaled inputs count K in storage bytes (an E2M1 byte holds 2 elements).
template <int IN, int BK16>
inline constexpr int bk_of = (IN == DT_F8E4M3 || IN == DT_F8E5M2 || IN == DT_MX_E4M3 ||
                              IN == DT_MX_E5M2 || IN == DT_MX_E2M1)
                                 ? 2 * BK16
                                 : BK16;

template <int IN, int OUT, bool TB, int id> struct CfgOf;
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D256x256x64_S2> {
    using type = Cfg<IN, OUT, TB, 256, 256, bk_of<IN, 64>, 2, 2, 2, true>;
};
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D256x256x32_S4> {
    using type = Cfg<IN, OUT, TB, 256, 256, bk_of<IN, 32>, 2, 2, 4, true>;
};
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D256x256x32_S5> {
    using type = Cfg<IN, OUT, TB, 256, 256, bk_of<IN, 32>, 2, 2, 5, true>;
};
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D256x256x32_S4_I> {
    using type = Cfg<IN, OUT, TB, 256, 256, bk_of<IN, 32>, 2, 2, 4, true, true>;
};
// d256x256x64_s2 contracted with 16x16x32 MFMAs (8 x 8 blocks per wave instead
// of 4 x 4): 16-bit inputs only.  A comparison variant: the 16x16 form draws
// less power per MAC, but the interleaved pipeline needs one MFMA k-step per
// 32-k step with it, and the compiler then shuffles its 64 accumulator
// tuples every step.
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D256x256x64_S2_16> {
    using type = Cfg<IN, OUT, TB, 256, 256, bk_of<IN, 64>, 2, 2, 2, true, false, 16>;
};
// The interleaved four-stage tile with 16x16x32 MFMA blocks (16-bit inputs):
// one MFMA k step per 32-k step, one fragment set reloaded in place.  The
// large-shape tile that plan selection takes for 16-bit inputs.  Built in its
// own units (inst_i16.hip), with the matrix instructions in their VGPR form.
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D256x256x32_S4_I16> {
    using type = Cfg<IN, OUT, TB, 256, 256, bk_of<IN, 32>, 2, 2, 4, true, true, 16>;
};
// The same tile 192 columns wide (waves of 128 x 96, 8 x 6 blocks), for B
// stored (N,K): the narrower last round of a two-region grid, where whole
// 256x256 rounds leave a partial one (4096 x 7168: 256 tiles of 256 x 256,
// then 256 of 256 x 192 instead of 192 more of 256 x 256).
template <int IN, int OUT> struct CfgOf<IN, OUT, true, CFG_D256x192x32_S4_I16> {
    using type = Cfg<IN, OUT, true, 256, 192, bk_of<IN, 32>, 2, 2, 4, true, true, 16>;
};
// The 16x16-block tile as a persistent kernel whose workgroups stream the K
// steps of their tiles through one ring, fetching each next tile's first
// steps during the current tile's last ones (16-bit inputs; M, N >= 256, K a
// multiple of 32 with at least 4 steps).
// The 16x16-block tile with eight waves (2 x 4, waves of 128 x 64): two waves
// per SIMD, so that one issues matrix instructions while the other waits at a
// barrier or for its fragments.  The large-shape tile plan selection takes for
// 16-bit inputs (measured on MI355X against the four-wave tile, same bits:
// 8192^3 fp16 0.5-2.3 % faster, 4097 x 3001 x 5003 4 %, whole 256 x 256 tiles
// of 4096 x 7168 x 4096 bf16 4.7 %).
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D256x256x32_S4_I16W8> {
    using type = Cfg<IN, OUT, TB, 256, 256, bk_of<IN, 32>, 2, 4, 4, true, true, 16>;
};
// Its narrower last round in a two-region grid (B stored (N,K); comparison
// build): 128 x 384 tiles of eight waves side by side (waves of 128 x 48, 8 x 3
// blocks), the same 128 KiB ring and one A and three B copies per thread a
// step.  A 256 x 192 tile has no whole copy count over 512 threads (768 B
// chunks a step); this one covers the same 49152 outputs.  Measured on
// MI355X (bf16 4096 x 7168 x 4096, fp32 C, one box): the eight-wave grid
// 187.7 us against the four-wave one's 182.4; its round runs at 0.74 of the
// 256 x 256 tile's rate per flop (each A fragment is read by all eight waves).
template <int IN, int OUT> struct CfgOf<IN, OUT, true, CFG_D128x384x32_S4_I16W8> {
    using type = Cfg<IN, OUT, true, 128, 384, bk_of<IN, 32>, 1, 8, 4, true, true, 16>;
};
// The eight-wave tile with its last, partial round split along K (stream-K;
// comparison build, gemm_relu_ws with GEMM_RELU_FORCE_CONFIG only): whole
// rounds of one workgroup per tile, then one workgroup per CU taking an equal
// share of the remaining tiles' K steps, with fp32 partials in the caller's
// workspace.  Measured on MI355X (one box): 4097 x 3001 x 5003 195.4 us against
// 125.5 for whole tiles (130.0 with one whole tile per unit, so the exchange of
// the 256 KiB partials costs ~65 us: ~190 MiB of device-scope traffic at
// ~3 TB/s), bf16 4096 x 7168 x 4096 219.7 against 182.4.
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D256x256x32_S4_I16W8SK> {
    using type = Cfg<IN, OUT, TB, 256, 256, bk_of<IN, 32>, 2, 4, 4, true, true, 16, false, true>;
};
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D256x256x32_S4_I16P> {
    using type = Cfg<IN, OUT, TB, 256, 256, bk_of<IN, 32>, 2, 2, 4, true, true, 16, true>;
};
// The 32x32-block interleaved tile as a persistent kernel: at most one workgroup
// per CU, each looping over its tiles (the Ascend version's T.Persistent).
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D256x256x32_S4_IP> {
    using type = Cfg<IN, OUT, TB, 256, 256, bk_of<IN, 32>, 2, 2, 4, true, true, 32, true>;
};
// The 32x32-block interleaved tile with its last round split along K (stream-K):
// the tiles that do not fill a whole round of CUs share their K steps out
// over all of them.
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D256x256x32_S4_ISK> {
    using type = Cfg<IN, OUT, TB, 256, 256, bk_of<IN, 32>, 2, 2, 4, true, true, 32, false, true>;
};
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D256x256x32_S4_W8I> {
    using type = Cfg<IN, OUT, TB, 256, 256, bk_of<IN, 32>, 2, 4, 4, true, true>;
};
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D256x256x32_S5_W8I> {
    using type = Cfg<IN, OUT, TB, 256, 256, bk_of<IN, 32>, 2, 4, 5, true, true>;
};
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D256x256x64_S2_W8> {
    using type = Cfg<IN, OUT, TB, 256, 256, bk_of<IN, 64>, 2, 4, 2, true>;
};
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D128x128x64_S3> {
    using type = Cfg<IN, OUT, TB, 128, 128, bk_of<IN, 64>, 2, 2, 3, true>;
};
// Skinny shapes with a workspace: 64 x 128 tiles (waves of 32 x 64), each
// tile's K range cut into parts taken by separate workgroups, which publish
// fp32 partial tiles; the last part of a tile to finish sums them, applies the
// ReLU and stores C.  A part reads 256-byte pieces of many consecutive (K,N) B
// rows, which HBM serves almost at the rate of contiguous reads, where
// whole-K 64-column tiles read 128-byte pieces of every row.
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D64x128x64_S4_SPLITK> {
    using type = Cfg<IN, OUT, TB, 64, 128, bk_of<IN, 64>, 2, 2, 4, true, false, 32, false, false, true>;
};
// Comparison variants of the K-split tile: 256 columns (512-byte row pieces),
// 128-element steps, and a three-stage ring small enough for two workgroups
// per CU.
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D64x256x64_S3_SPLITK> {
    using type = Cfg<IN, OUT, TB, 64, 256, bk_of<IN, 64>, 2, 2, 3, true, false, 32, false, false, true>;
};
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D64x128x128_S3_SPLITK> {
    using type = Cfg<IN, OUT, TB, 64, 128, bk_of<IN, 128>, 2, 2, 3, true, false, 32, false, false, true>;
};
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D64x128x64_S3_SPLITK> {
    using type = Cfg<IN, OUT, TB, 64, 128, bk_of<IN, 64>, 2, 2, 3, true, false, 32, false, false, true>;
};
// Two-stage 128x128: the smaller tile of the block-scaled inputs.
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D128x128x64_S2> {
    using type = Cfg<IN, OUT, TB, 128, 128, bk_of<IN, 64>, 2, 2, 2, true>;
};
// Two-stage 256x128 (waves of 128x64): fewer fragment registers than 256x256
// for the block-scaled inputs, whose per-lane scales need registers too.
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D256x128x64_S2> {
    using type = Cfg<IN, OUT, TB, 256, 128, bk_of<IN, 64>, 2, 2, 2, true>;
};
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D64x64x64_S4> {
    using type = Cfg<IN, OUT, TB, 64, 64, bk_of<IN, 64>, 2, 2, 4, true>;
};
// Skinny / memory-bound problems: 2 waves, a long BK and 96 KiB of LDS, so one
// workgroup per CU and twice as many workgroups as the 64x64 tile.
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D64x32x128_S4> {
    using type = Cfg<IN, OUT, TB, 64, 32, bk_of<IN, 128>, 2, 1, 4, true>;
};
// Skinny problems, the other way round: 32 rows by 64 columns, so each k row
// of a (K,N) B tile is one whole 128-byte line; two waves side by side in N.
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_D32x64x128_S4> {
    using type = Cfg<IN, OUT, TB, 32, 64, bk_of<IN, 128>, 1, 2, 4, true>;
};
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_G128x128x64> {
    using type = Cfg<IN, OUT, TB, 128, 128, bk_of<IN, 64>, 2, 2, 2, false>;
};
template <int IN, int OUT, bool TB> struct CfgOf<IN, OUT, TB, CFG_G64x64x64> {
    using type = Cfg<IN, OUT, TB, 64, 64, bk_of<IN, 64>, 2, 2, 2, false>;
};

typedef hipError_t (*LaunchFn)(const KernelArgs& args, int grid, hipStream_t stream);

template <class C>
hipError_t launch_one(const KernelArgs& args, int grid, hipStream_t stream)
{
    void* params[] = {const_cast<KernelArgs*>(&args)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_relu_kernel<C>), dim3(grid),
                           dim3(C::NTHREADS), params, 0, stream);
}

// A two-region grid: whole rounds of C1 tiles, then a round of C2 tiles.
template <class C1, class C2>
hipError_t launch_two(const KernelArgs& args, int grid, hipStream_t stream)
{
    void* params[] = {const_cast<KernelArgs*>(&args)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_relu_kernel_2r<C1, C2>), dim3(grid),
                           dim3(C1::NTHREADS), params, 0, stream);
}

// The launcher of a comparison configuration: instantiated only in a build
// that holds them.
template <class C>
LaunchFn comparison_launcher()
{
    if constexpr (kComparisonBuilt)
        return &launch_one<C>;
    else
        return nullptr;
}

// One table per (input dtype, transB); defined in the instantiation units.
LaunchFn launcher_f16_nn(int out_dt, int cfg);
LaunchFn launcher_f16_nt(int out_dt, int cfg);
LaunchFn launcher_bf16_nn(int out_dt, int cfg);
LaunchFn launcher_bf16_nt(int out_dt, int cfg);
LaunchFn launcher_f8e4m3_nn(int out_dt, int cfg);
LaunchFn launcher_f8e4m3_nt(int out_dt, int cfg);
LaunchFn launcher_f8e5m2_nn(int out_dt, int cfg);
LaunchFn launcher_f8e5m2_nt(int out_dt, int cfg);
LaunchFn launcher_mx_e4m3(int out_dt, int cfg);
LaunchFn launcher_mx_e5m2(int out_dt, int cfg);
LaunchFn launcher_mx_e2m1(int out_dt, int cfg);
// the 16x16-block interleaved tiles for a 16-bit input type (inst_i16.hip):
// 256 x 256 with four or eight waves (either B layout); 256 x 192 (four waves)
// and 128 x 384 (eight waves) for B stored (N,K); and the two-region grids
// (B stored (N,K)) whose narrower round is cfg2, one of those two
LaunchFn launcher_i16(int in_dt, int out_dt, bool transB);
LaunchFn launcher_i16_192(int in_dt, int out_dt);
LaunchFn launcher_i16_384(int in_dt, int out_dt);
LaunchFn launcher_i16p(int in_dt, int out_dt, bool transB);
LaunchFn launcher_i16w8(int in_dt, int out_dt, bool transB);
LaunchFn launcher_i16w8sk(int in_dt, int out_dt, bool transB);
LaunchFn launcher_i16_2r(int in_dt, int out_dt, int cfg2);

// Configurations built for 8-bit inputs: the ones plan selection can choose
// (the 16-bit comparison variants are not instantiated for them).
inline bool fp8_config(int cfg)
{
    return cfg == CFG_D256x256x32_S4_I || cfg == CFG_D256x256x32_S4_ISK ||
           cfg == CFG_D128x128x64_S3 || cfg == CFG_D64x64x64_S4 || cfg == CFG_D32x64x128_S4 ||
           cfg == CFG_D64x32x128_S4 || cfg == CFG_G128x128x64 || cfg == CFG_G64x64x64 ||
           cfg == CFG_D64x128x64_S4_SPLITK || cfg == CFG_D64x256x64_S3_SPLITK ||
           cfg == CFG_D64x128x128_S3_SPLITK || cfg == CFG_D64x128x64_S3_SPLITK;
}

}  // namespace gemm_relu_hip

// Body of an instantiation unit: every configuration for one (IN, TRANS_B)
// and the three output types.
#define GEMM_RELU_DEFINE_LAUNCHER(FN, IN, TB)                                              \
    namespace gemm_relu_hip {                                                              \
    template <int OUT>                                                                     \
    static LaunchFn FN##_out(int cfg)                                                      \
    {                                                                                      \
        switch (cfg) {                                                                     \
        case CFG_D256x256x64_S2:                                                           \
            return comparison_launcher<typename CfgOf<IN, OUT, TB, CFG_D256x256x64_S2>::type>(); \
        case CFG_D256x256x32_S4:                                                           \
            return comparison_launcher<typename CfgOf<IN, OUT, TB, CFG_D256x256x32_S4>::type>(); \
        case CFG_D256x256x32_S5:                                                           \
            return comparison_launcher<typename CfgOf<IN, OUT, TB, CFG_D256x256x32_S5>::type>(); \
        case CFG_D256x256x32_S4_I:                                                         \
            return &launch_one<typename CfgOf<IN, OUT, TB, CFG_D256x256x32_S4_I>::type>;   \
        case CFG_D256x256x64_S2_16:                                                        \
            return comparison_launcher<typename CfgOf<IN, OUT, TB, CFG_D256x256x64_S2_16>::type>(); \
        case CFG_D256x256x32_S4_I16:                                                       \
            return launcher_i16(IN, OUT, TB);                                              \
        case CFG_D256x192x32_S4_I16:                                                       \
            return TB ? launcher_i16_192(IN, OUT) : nullptr;                               \
        case CFG_D256x256x32_S4_I16P:                                                      \
            return launcher_i16p(IN, OUT, TB);                                             \
        case CFG_D256x256x32_S4_I16W8:                                                     \
            return launcher_i16w8(IN, OUT, TB);                                            \
        case CFG_D256x256x32_S4_I16W8SK:                                                   \
            return launcher_i16w8sk(IN, OUT, TB);                                          \
        case CFG_D128x384x32_S4_I16W8:                                                     \
            return TB ? launcher_i16_384(IN, OUT) : nullptr;                               \
        case CFG_D256x256x32_S4_IP:                                                        \
            return comparison_launcher<typename CfgOf<IN, OUT, TB, CFG_D256x256x32_S4_IP>::type>(); \
        case CFG_D256x256x32_S4_ISK:                                                       \
            return comparison_launcher<typename CfgOf<IN, OUT, TB, CFG_D256x256x32_S4_ISK>::type>(); \
        case CFG_D256x256x32_S4_W8I:                                                       \
            return comparison_launcher<typename CfgOf<IN, OUT, TB, CFG_D256x256x32_S4_W8I>::type>(); \
        case CFG_D256x256x32_S5_W8I:                                                       \
            return comparison_launcher<typename CfgOf<IN, OUT, TB, CFG_D256x256x32_S5_W8I>::type>(); \
        case CFG_D256x256x64_S2_W8:                                                        \
            return comparison_launcher<typename CfgOf<IN, OUT, TB, CFG_D256x256x64_S2_W8>::type>(); \
        case CFG_D128x128x64_S3:                                                           \
            return &launch_one<typename CfgOf<IN, OUT, TB, CFG_D128x128x64_S3>::type>;     \
        case CFG_D128x128x64_S2:                                                           \
            return &launch_one<typename CfgOf<IN, OUT, TB, CFG_D128x128x64_S2>::type>;     \
        case CFG_D64x64x64_S4:                                                             \
            return &launch_one<typename CfgOf<IN, OUT, TB, CFG_D64x64x64_S4>::type>;       \
        case CFG_D64x32x128_S4:                                                            \
            return &launch_one<typename CfgOf<IN, OUT, TB, CFG_D64x32x128_S4>::type>;      \
        case CFG_D32x64x128_S4:                                                            \
            return &launch_one<typename CfgOf<IN, OUT, TB, CFG_D32x64x128_S4>::type>;      \
        case CFG_D64x128x64_S4_SPLITK:                                                     \
            return &launch_one<typename CfgOf<IN, OUT, TB, CFG_D64x128x64_S4_SPLITK>::type>; \
        case CFG_D64x256x64_S3_SPLITK:                                                     \
            return comparison_launcher<typename CfgOf<IN, OUT, TB, CFG_D64x256x64_S3_SPLITK>::type>(); \
        case CFG_D64x128x128_S3_SPLITK:                                                    \
            return comparison_launcher<typename CfgOf<IN, OUT, TB, CFG_D64x128x128_S3_SPLITK>::type>(); \
        case CFG_D64x128x64_S3_SPLITK:                                                     \
            return comparison_launcher<typename CfgOf<IN, OUT, TB, CFG_D64x128x64_S3_SPLITK>::type>(); \
        case CFG_G128x128x64:                                                              \
            return &launch_one<typename CfgOf<IN, OUT, TB, CFG_G128x128x64>::type>;        \
        case CFG_G64x64x64:                                                                \
            return &launch_one<typename CfgOf<IN, OUT, TB, CFG_G64x64x64>::type>;          \
        default:                                                                           \
            return nullptr;                                                                \
        }                                                                                  \
    }                                                                                      \
    LaunchFn FN(int out_dt, int cfg)                                                       \
    {                                                                                      \
        switch (out_dt) {                                                                  \
        case DT_F16: return FN##_out<DT_F16>(cfg);                                         \
        case DT_BF16: return FN##_out<DT_BF16>(cfg);                                       \
        case DT_F32: return FN##_out<DT_F32>(cfg);                                         \
        default: return nullptr;                                                           \
        }                                                                                  \
    }                                                                                      \
    }

// Body of an 8-bit instantiation unit: the configurations fp8_config() names.
#define GEMM_RELU_DEFINE_LAUNCHER_FP8(FN, IN, TB)                                          \
    namespace gemm_relu_hip {                                                              \
    template <int OUT>                                                                     \
    static LaunchFn FN##_out(int cfg)                                                      \
    {                                                                                      \
        switch (cfg) {                                                                     \
        case CFG_D256x256x32_S4_I:                                                         \
            return &launch_one<typename CfgOf<IN, OUT, TB, CFG_D256x256x32_S4_I>::type>;   \
        case CFG_D256x256x32_S4_ISK:                                                       \
            return comparison_launcher<typename CfgOf<IN, OUT, TB, CFG_D256x256x32_S4_ISK>::type>(); \
        case CFG_D128x128x64_S3:                                                           \
            return &launch_one<typename CfgOf<IN, OUT, TB, CFG_D128x128x64_S3>::type>;     \
        case CFG_D128x128x64_S2:                                                           \
            return &launch_one<typename CfgOf<IN, OUT, TB, CFG_D128x128x64_S2>::type>;     \
        case CFG_D64x64x64_S4:                                                             \
            return &launch_one<typename CfgOf<IN, OUT, TB, CFG_D64x64x64_S4>::type>;       \
        case CFG_D64x32x128_S4:                                                            \
            return &launch_one<typename CfgOf<IN, OUT, TB, CFG_D64x32x128_S4>::type>;      \
        case CFG_D32x64x128_S4:                                                            \
            return &launch_one<typename CfgOf<IN, OUT, TB, CFG_D32x64x128_S4>::type>;      \
        case CFG_D64x128x64_S4_SPLITK:                                                     \
            return &launch_one<typename CfgOf<IN, OUT, TB, CFG_D64x128x64_S4_SPLITK>::type>; \
        case CFG_D64x256x64_S3_SPLITK:                                                     \
            return comparison_launcher<typename CfgOf<IN, OUT, TB, CFG_D64x256x64_S3_SPLITK>::type>(); \
        case CFG_D64x128x128_S3_SPLITK:                                                    \
            return comparison_launcher<typename CfgOf<IN, OUT, TB, CFG_D64x128x128_S3_SPLITK>::type>(); \
        case CFG_D64x128x64_S3_SPLITK:                                                     \
            return comparison_launcher<typename CfgOf<IN, OUT, TB, CFG_D64x128x64_S3_SPLITK>::type>(); \
        case CFG_G128x128x64:                                                              \
            return &launch_one<typename CfgOf<IN, OUT, TB, CFG_G128x128x64>::type>;        \
        case CFG_G64x64x64:                                                                \
            return &launch_one<typename CfgOf<IN, OUT, TB, CFG_G64x64x64>::type>;          \
        default:                                                                           \
            return nullptr;                                                                \
        }                                                                                  \
    }                                                                                      \
    LaunchFn FN(int out_dt, int cfg)                                                       \
    {                                                                                      \
        switch (out_dt) {                                                                  \
        case DT_F16: return FN##_out<DT_F16>(cfg);                                         \
        case DT_BF16: return FN##_out<DT_BF16>(cfg);                                       \
        case DT_F32: return FN##_out<DT_F32>(cfg);                                         \
        default: return nullptr;                                                           \
        }                                                                                  \
    }                                                                                      \
    }

// Body of a block-scaled instantiation unit: B stored (N,K), the two-stage
// direct configurations.
#define GEMM_RELU_DEFINE_LAUNCHER_MX(FN, IN)                                               \
    namespace gemm_relu_hip {                                                              \
    template <int OUT>                                                                     \
    static LaunchFn FN##_out(int cfg)                                                      \
    {                                                                                      \
        switch (cfg) {                                                                     \
        case CFG_D256x256x32_S4_I:                                                         \
            return &launch_one<typename CfgOf<IN, OUT, true, CFG_D256x256x32_S4_I>::type>; \
        case CFG_D256x256x64_S2:                                                           \
            return comparison_launcher<typename CfgOf<IN, OUT, true, CFG_D256x256x64_S2>::type>(); \
        case CFG_D128x128x64_S2:                                                           \
            return &launch_one<typename CfgOf<IN, OUT, true, CFG_D128x128x64_S2>::type>;   \
        case CFG_D256x128x64_S2:                                                           \
            return comparison_launcher<typename CfgOf<IN, OUT, true, CFG_D256x128x64_S2>::type>(); \
        default:                                                                           \
            return nullptr;                                                                \
        }                                                                                  \
    }                                                                                      \
    LaunchFn FN(int out_dt, int cfg)                                                       \
    {                                                                                      \
        switch (out_dt) {                                                                  \
        case DT_F16: return FN##_out<DT_F16>(cfg);                                         \
        case DT_BF16: return FN##_out<DT_BF16>(cfg);                                       \
        case DT_F32: return FN##_out<DT_F32>(cfg);                                         \
        default: return nullptr;                                                           \
        }                                                                                  \
    }                                                                                      \
    }
