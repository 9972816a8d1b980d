// Instantiations of the 2:4 sparse GEMM + ReLU kernel: 16-bit inputs, both B
// layouts, every output type.
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

template <int IN, bool TB>
static SpLaunchFn sp_out(int out_dt)
{
    switch (out_dt) {
    case DT_F16: return &launch_sp<SpCfg<IN, DT_F16, TB>>;
    case DT_BF16: return &launch_sp<SpCfg<IN, DT_BF16, TB>>;
    case DT_F32: return &launch_sp<SpCfg<IN, DT_F32, TB>>;
    default: return nullptr;
    }
}

SpLaunchFn launcher_sp(int in_dt, int out_dt, int transB)
{
    if (in_dt == DT_F16) return transB ? sp_out<DT_F16, true>(out_dt) : sp_out<DT_F16, false>(out_dt);
    if (in_dt == DT_BF16) return transB ? sp_out<DT_BF16, true>(out_dt) : sp_out<DT_BF16, false>(out_dt);
    return nullptr;
}

}  // namespace gemm_relu_hip
