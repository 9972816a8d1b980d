// Instantiations of the 2:4 sparse GEMM + ReLU kernel: 16-bit inputs, both B
// layouts, every output type.
#include "configs.hpp"
#include "gemm_sp_relu_kernel.hpp"

namespace gemm_relu_hip {

typedef hipError_t (*SpLaunchFn)(const SpArgs& args, int grid, hipStream_t stream);

template <class C>
static hipError_t launch_sp(const SpArgs& args, int grid, hipStream_t stream)
{
    void* params[] = {const_cast<SpArgs*>(&args)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_sp_relu_kernel<C>), dim3(grid),
                           dim3(C::NTHREADS), params, 0, stream);
}

// The launcher of a comparison variant: instantiated only in a build that holds them.
template <class C>
static SpLaunchFn sp_comparison()
{
    if constexpr (kComparisonBuilt)
        return &launch_sp<C>;
    else
        return nullptr;
}

// variant 1: 2 x 4 waves (two per SIMD); 0: 2 x 2 waves (comparison build;
// measured on MI355X at 8192^3 fp16: 651.9 against 589.3 us, the same bits)
template <int IN, bool TB, int WN>
static SpLaunchFn sp_out(int out_dt)
{
    if constexpr (WN == 4) {
        switch (out_dt) {
        case DT_F16: return &launch_sp<SpCfg<IN, DT_F16, TB, 3, WN>>;
        case DT_BF16: return &launch_sp<SpCfg<IN, DT_BF16, TB, 3, WN>>;
        case DT_F32: return &launch_sp<SpCfg<IN, DT_F32, TB, 3, WN>>;
        default: return nullptr;
        }
    } else {
        switch (out_dt) {
        case DT_F16: return sp_comparison<SpCfg<IN, DT_F16, TB, 3, WN>>();
        case DT_BF16: return sp_comparison<SpCfg<IN, DT_BF16, TB, 3, WN>>();
        case DT_F32: return sp_comparison<SpCfg<IN, DT_F32, TB, 3, WN>>();
        default: return nullptr;
        }
    }
}

template <int WN>
static SpLaunchFn sp_in(int in_dt, int out_dt, int transB)
{
    if (in_dt == DT_F16) return transB ? sp_out<DT_F16, true, WN>(out_dt) : sp_out<DT_F16, false, WN>(out_dt);
    if (in_dt == DT_BF16) return transB ? sp_out<DT_BF16, true, WN>(out_dt) : sp_out<DT_BF16, false, WN>(out_dt);
    return nullptr;
}

SpLaunchFn launcher_sp(int in_dt, int out_dt, int transB, int variant)
{
    return variant == 0 ? sp_in<2>(in_dt, out_dt, transB) : sp_in<4>(in_dt, out_dt, transB);
}

}  // namespace gemm_relu_hip
