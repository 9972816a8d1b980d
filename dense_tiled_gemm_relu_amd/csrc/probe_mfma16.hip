// MFMA-only throughput of v_mfma_f32_16x16x32_f16 on random operands (kind 5
// of probe_mfma_rate): the ceiling of the GEMM's 16x16-block contraction on a
// power-limited chip.  Diagnostic only; built into the probe library.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "gemm_relu_kernel.hpp"

using namespace gemm_relu_hip;

namespace {

constexpr int kThreads = 256;
constexpr int kOperandRegs = 8;     // 4 A + 4 B fragments per lane

// kind 5: v_mfma_f32_16x16x32_f16, the 64 MFMAs of one step of a 128x128
// wave tile in 16x16 blocks (8 x 8 blocks, the same 4 + 4 operand registers
// used twice each).  One step per loop iteration, so each accumulator is
// updated once per iteration and stays in its registers.
__global__ void __launch_bounds__(kThreads, 1)
k_mfma16_rate(const unsigned char* src, float* out, unsigned long long* ticks, int steps)
{
    const int tid = threadIdx.x;
    constexpr int OPB = 16;
    const size_t base = ((size_t)blockIdx.x * kOperandRegs * kThreads + tid) * OPB;
    f16x8_t a[4], b[4];
    for (int i = 0; i < 4; ++i) {
        __builtin_memcpy(&a[i], src + base + (size_t)i * kThreads * OPB, OPB);
        __builtin_memcpy(&b[i], src + base + (size_t)(4 + i) * kThreads * OPB, OPB);
    }
    f32x4_t acc[64];
    for (int i = 0; i < 64; ++i)
        for (int r = 0; r < 4; ++r) acc[i][r] = 0.0f;
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    for (int it = 0; it < steps; ++it) {         // one 128x128x32 wave step, as a kind-0 step
#pragma unroll
        for (int p = 0; p < 64; ++p) {
            const int j = p / 8, ii = p % 8, i = (j & 1) ? 7 - ii : ii;
            acc[8 * j + i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[j % 4], a[i % 4], acc[8 * j + i], 0, 0, 0);
        }
        __builtin_amdgcn_s_barrier();
    }
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.0f;
    for (int i = 0; i < 64; ++i)
        for (int r = 0; r < 4; ++r) s += acc[i][r];
    out[(size_t)blockIdx.x * kThreads + tid] = s;
    if (tid == 0) {
        ticks[2 * (size_t)blockIdx.x] = c1 - c0;
        ticks[2 * (size_t)blockIdx.x + 1] = r1 - r0;
    }
}

}  // namespace

hipError_t launch_mfma16_rate(const unsigned char* src, float* out, unsigned long long* ticks,
                              int blocks, int steps, hipStream_t stream)
{
    hipLaunchKernelGGL(k_mfma16_rate, dim3(blocks), dim3(kThreads), 0, stream, src, out, ticks, steps);
    return hipGetLastError();
}
