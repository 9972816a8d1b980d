// Instantiations of the interleaved 256x256 tile with 16x16x32 MFMA blocks,
// 16-bit inputs, both B layouts, every output type, with four and with eight
// waves; its narrower forms (256x192, four waves; 128x384, eight waves) and the
// two-region grids for B stored (N,K).  Kept apart from the other
// configurations because this unit is compiled with the matrix instructions in
// their VGPR form, which keeps the 64 small accumulators in place.
#include "configs.hpp"

namespace gemm_relu_hip {

template <int IN, bool TB>
static LaunchFn i16_out(int out_dt)
{
    switch (out_dt) {
    case DT_F16: return &launch_one<typename CfgOf<IN, DT_F16, TB, CFG_D256x256x32_S4_I16>::type>;
    case DT_BF16: return &launch_one<typename CfgOf<IN, DT_BF16, TB, CFG_D256x256x32_S4_I16>::type>;
    case DT_F32: return &launch_one<typename CfgOf<IN, DT_F32, TB, CFG_D256x256x32_S4_I16>::type>;
    default: return nullptr;
    }
}

LaunchFn launcher_i16(int in_dt, int out_dt, bool transB)
{
    if (in_dt == DT_F16) return transB ? i16_out<DT_F16, true>(out_dt) : i16_out<DT_F16, false>(out_dt);
    if (in_dt == DT_BF16) return transB ? i16_out<DT_BF16, true>(out_dt) : i16_out<DT_BF16, false>(out_dt);
    return nullptr;
}

template <int IN, int OUT>
using Big = typename CfgOf<IN, OUT, true, CFG_D256x256x32_S4_I16>::type;
template <int IN, int OUT>
using Narrow = typename CfgOf<IN, OUT, true, CFG_D256x192x32_S4_I16>::type;

template <int IN>
static LaunchFn i16_192_out(int out_dt)
{
    switch (out_dt) {
    case DT_F16: return &launch_one<Narrow<IN, DT_F16>>;
    case DT_BF16: return &launch_one<Narrow<IN, DT_BF16>>;
    case DT_F32: return &launch_one<Narrow<IN, DT_F32>>;
    default: return nullptr;
    }
}

template <int IN, int OUT>
using Big8 = typename CfgOf<IN, OUT, true, CFG_D256x256x32_S4_I16W8>::type;
template <int IN, int OUT>
using Narrow8 = typename CfgOf<IN, OUT, true, CFG_D128x384x32_S4_I16W8>::type;

template <int IN>
static LaunchFn i16_384_out(int out_dt)
{
    switch (out_dt) {
    case DT_F16: return comparison_launcher<Narrow8<IN, DT_F16>>();
    case DT_BF16: return comparison_launcher<Narrow8<IN, DT_BF16>>();
    case DT_F32: return comparison_launcher<Narrow8<IN, DT_F32>>();
    default: return nullptr;
    }
}

template <int IN>
static LaunchFn i16_2r_out(int out_dt)
{
    switch (out_dt) {
    case DT_F16: return &launch_two<Big<IN, DT_F16>, Narrow<IN, DT_F16>>;
    case DT_BF16: return &launch_two<Big<IN, DT_BF16>, Narrow<IN, DT_BF16>>;
    case DT_F32: return &launch_two<Big<IN, DT_F32>, Narrow<IN, DT_F32>>;
    default: return nullptr;
    }
}

// the launcher of the eight-wave two-region grid (comparison build)
template <class C1, class C2>
static LaunchFn comparison_two()
{
    if constexpr (kComparisonBuilt)
        return &launch_two<C1, C2>;
    else
        return nullptr;
}

template <int IN>
static LaunchFn i16w8_2r_out(int out_dt)
{
    switch (out_dt) {
    case DT_F16: return comparison_two<Big8<IN, DT_F16>, Narrow8<IN, DT_F16>>();
    case DT_BF16: return comparison_two<Big8<IN, DT_BF16>, Narrow8<IN, DT_BF16>>();
    case DT_F32: return comparison_two<Big8<IN, DT_F32>, Narrow8<IN, DT_F32>>();
    default: return nullptr;
    }
}

template <int IN, bool TB>
static LaunchFn i16p_out(int out_dt)
{
    switch (out_dt) {
    case DT_F16: return comparison_launcher<typename CfgOf<IN, DT_F16, TB, CFG_D256x256x32_S4_I16P>::type>();
    case DT_BF16: return comparison_launcher<typename CfgOf<IN, DT_BF16, TB, CFG_D256x256x32_S4_I16P>::type>();
    case DT_F32: return comparison_launcher<typename CfgOf<IN, DT_F32, TB, CFG_D256x256x32_S4_I16P>::type>();
    default: return nullptr;
    }
}

LaunchFn launcher_i16p(int in_dt, int out_dt, bool transB)
{
    if (in_dt == DT_F16) return transB ? i16p_out<DT_F16, true>(out_dt) : i16p_out<DT_F16, false>(out_dt);
    if (in_dt == DT_BF16) return transB ? i16p_out<DT_BF16, true>(out_dt) : i16p_out<DT_BF16, false>(out_dt);
    return nullptr;
}

template <int IN, bool TB>
static LaunchFn i16w8_out(int out_dt)
{
    switch (out_dt) {
    case DT_F16: return &launch_one<typename CfgOf<IN, DT_F16, TB, CFG_D256x256x32_S4_I16W8>::type>;
    case DT_BF16: return &launch_one<typename CfgOf<IN, DT_BF16, TB, CFG_D256x256x32_S4_I16W8>::type>;
    case DT_F32: return &launch_one<typename CfgOf<IN, DT_F32, TB, CFG_D256x256x32_S4_I16W8>::type>;
    default: return nullptr;
    }
}

LaunchFn launcher_i16w8(int in_dt, int out_dt, bool transB)
{
    if (in_dt == DT_F16) return transB ? i16w8_out<DT_F16, true>(out_dt) : i16w8_out<DT_F16, false>(out_dt);
    if (in_dt == DT_BF16) return transB ? i16w8_out<DT_BF16, true>(out_dt) : i16w8_out<DT_BF16, false>(out_dt);
    return nullptr;
}

template <int IN, bool TB>
static LaunchFn i16w8sk_out(int out_dt)
{
    switch (out_dt) {
    case DT_F16: return comparison_launcher<typename CfgOf<IN, DT_F16, TB, CFG_D256x256x32_S4_I16W8SK>::type>();
    case DT_BF16: return comparison_launcher<typename CfgOf<IN, DT_BF16, TB, CFG_D256x256x32_S4_I16W8SK>::type>();
    case DT_F32: return comparison_launcher<typename CfgOf<IN, DT_F32, TB, CFG_D256x256x32_S4_I16W8SK>::type>();
    default: return nullptr;
    }
}

LaunchFn launcher_i16w8sk(int in_dt, int out_dt, bool transB)
{
    if (in_dt == DT_F16) return transB ? i16w8sk_out<DT_F16, true>(out_dt) : i16w8sk_out<DT_F16, false>(out_dt);
    if (in_dt == DT_BF16) return transB ? i16w8sk_out<DT_BF16, true>(out_dt) : i16w8sk_out<DT_BF16, false>(out_dt);
    return nullptr;
}

LaunchFn launcher_i16_192(int in_dt, int out_dt)
{
    if (in_dt == DT_F16) return i16_192_out<DT_F16>(out_dt);
    if (in_dt == DT_BF16) return i16_192_out<DT_BF16>(out_dt);
    return nullptr;
}

LaunchFn launcher_i16_384(int in_dt, int out_dt)
{
    if (in_dt == DT_F16) return i16_384_out<DT_F16>(out_dt);
    if (in_dt == DT_BF16) return i16_384_out<DT_BF16>(out_dt);
    return nullptr;
}

LaunchFn launcher_i16_2r(int in_dt, int out_dt, int cfg2)
{
    if (cfg2 == CFG_D128x384x32_S4_I16W8) {
        if (in_dt == DT_F16) return i16w8_2r_out<DT_F16>(out_dt);
        if (in_dt == DT_BF16) return i16w8_2r_out<DT_BF16>(out_dt);
        return nullptr;
    }
    if (cfg2 != CFG_D256x192x32_S4_I16) return nullptr;
    if (in_dt == DT_F16) return i16_2r_out<DT_F16>(out_dt);
    if (in_dt == DT_BF16) return i16_2r_out<DT_BF16>(out_dt);
    return nullptr;
}

}  // namespace gemm_relu_hip
