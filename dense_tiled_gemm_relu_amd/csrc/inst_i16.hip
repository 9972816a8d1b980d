// Instantiations of the interleaved 256x256 tile with 16x16x32 MFMA blocks,
// 16-bit inputs, both B layouts, every output type.  Kept apart from the other
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

}  // namespace gemm_relu_hip
