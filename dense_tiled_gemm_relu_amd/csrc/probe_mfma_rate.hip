// MFMA-only throughput on random operands: the practical ceiling of the GEMM's
// contraction step on a power-limited chip.
//
// Each workgroup is 4 waves (one per SIMD, 512 registers each, one workgroup per
// CU).  Every wave repeats `steps` rounds of 32 independent MFMAs over 16
// accumulators and 4 + 4 operand registers: the MFMA stream of one step of a
// 128x128 wave tile, with no memory traffic and no LDS.  kind 0:
// v_mfma_f32_32x32x16_f16 (16-byte operands); kind 1:
// v_mfma_f32_32x32x64_f8f6f4 on E4M3 data (32-byte operands); kind 2:
// v_mfma_scale_f32_32x32x64_f8f6f4 on E2M1 data with unit E8M0 scales
// (16-byte operands); kind 3: the same scaled MFMA on E4M3 data (32-byte
// operands); kind 4: v_smfmac_f32_32x32x32_f16, the 2:4 sparse form (a 16-byte
// compressed operand, a 32-byte dense one, a fixed valid index word); kind 5:
// v_mfma_f32_16x16x32_f16 (16-byte operands), the same step as 64 MFMAs of
// 16x16 blocks.  The operands are the caller's random data, so the multiplier
// arrays toggle as they do in the GEMM; on MI355X this, not the instruction
// rate, sets the shader clock.  Wave 0 of each workgroup records the shader
// cycles (s_memtime) and 100 MHz reference ticks (s_memrealtime) of its loop.
// Diagnostic only; built into the probe library, not the product library.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "gemm_sp_relu_kernel.hpp"

using namespace gemm_relu_hip;

namespace {

constexpr int kThreads = 256;
constexpr int kOperandRegs = 8;     // 4 A + 4 B fragments per lane

template <int IN_DT>
__global__ void __launch_bounds__(kThreads, 1)
k_mfma_rate(const unsigned char* src, float* out, unsigned long long* ticks, int steps)
{
    using In = InTraits<IN_DT>;
    using Op = typename In::Op;
    const int tid = threadIdx.x;
    constexpr int OPB = In::OPB;      // operand bytes per lane
    const size_t base = ((size_t)blockIdx.x * kOperandRegs * kThreads + tid) * OPB;
    Op a[4], b[4];
    for (int i = 0; i < 4; ++i) {
        a[i] = Op{};
        b[i] = Op{};
        __builtin_memcpy(&a[i], src + base + (size_t)i * kThreads * OPB, OPB);
        __builtin_memcpy(&b[i], src + base + (size_t)(4 + i) * kThreads * OPB, OPB);
    }
    f32x16_t acc[16];
    for (int i = 0; i < 16; ++i)
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the timer reads have returned
    for (int it = 0; it < steps; ++it) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int p = 0; p < 16; ++p) {
                if constexpr (In::MX)
                    acc[p] = In::mfma_scaled(b[p / 4], a[p % 4], acc[p], 127, 127);
                else
                    acc[p] = In::mfma(b[p / 4], a[p % 4], acc[p]);
            }
        __builtin_amdgcn_s_barrier();
    }
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.0f;
    for (int i = 0; i < 16; ++i)
        for (int r = 0; r < 16; ++r) s += acc[i][r];
    out[(size_t)blockIdx.x * kThreads + tid] = s;     // keeps the MFMAs live
    if (tid == 0) {
        ticks[2 * (size_t)blockIdx.x] = c1 - c0;
        ticks[2 * (size_t)blockIdx.x + 1] = r1 - r0;
    }
}

// kind 4: the same loop on the sparse instruction; a[] takes the first 16
// bytes of its 32-byte slot.
__global__ void __launch_bounds__(kThreads, 1)
k_smfmac_rate(const unsigned char* src, float* out, unsigned long long* ticks, int steps)
{
    const int tid = threadIdx.x;
    constexpr int OPB = 32;
    const size_t base = ((size_t)blockIdx.x * kOperandRegs * kThreads + tid) * OPB;
    i32x4s_t a[4];
    i32x8_t b[4];
    for (int i = 0; i < 4; ++i) {
        __builtin_memcpy(&a[i], src + base + (size_t)i * kThreads * OPB, 16);
        __builtin_memcpy(&b[i], src + base + (size_t)(4 + i) * kThreads * OPB, 32);
    }
    // groups keep positions (0,1), (1,3), (0,2), (2,3): nibbles 4, 13, 8, 14
    const int idx = 0xE8D4;
    f32x16_t acc[16];
    for (int i = 0; i < 16; ++i)
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    for (int it = 0; it < steps; ++it) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int p = 0; p < 16; ++p)
                acc[p] = SpIn<DT_F16>::smfmac(a[p % 4], b[p / 4], acc[p], idx);
        __builtin_amdgcn_s_barrier();
    }
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.0f;
    for (int i = 0; i < 16; ++i)
        for (int r = 0; r < 16; ++r) s += acc[i][r];
    out[(size_t)blockIdx.x * kThreads + tid] = s;
    if (tid == 0) {
        ticks[2 * (size_t)blockIdx.x] = c1 - c0;
        ticks[2 * (size_t)blockIdx.x + 1] = r1 - r0;
    }
}

}  // namespace

// kind 5 lives in probe_mfma16.hip (built with the matrix instructions in their
// VGPR form, which keeps its 64 small accumulators in place)
hipError_t launch_mfma16_rate(const unsigned char* src, float* out, unsigned long long* ticks,
                              int blocks, int steps, hipStream_t stream);

// src: at least blocks * 8 * 256 * OPB bytes of input data (OPB = 16 for
// kind 0, fp16; 32 for kinds 1 and 3, E4M3; 16 for kind 2, packed E2M1; 32
// for kind 4, fp16); out: blocks * 256 floats; ticks:
// 2 * blocks values (shader cycles, reference ticks per workgroup).  Launches
// on `stream` without synchronising.  Returns 0, -1 on bad arguments, -3 on a
// launch failure.
extern "C" int probe_mfma_rate(const void* src, size_t src_bytes, void* out, void* ticks,
                               int blocks, int steps, int kind, void* stream)
{
    if (kind < 0 || kind > 5) return -1;
    const size_t opb = (kind == 1 || kind == 3 || kind == 4) ? 32 : 16;
    if (!src || !out || !ticks || blocks <= 0 || steps <= 0 ||
        src_bytes < (size_t)blocks * kOperandRegs * kThreads * opb)
        return -1;
    const hipStream_t st = (hipStream_t)stream;
    const unsigned char* s = (const unsigned char*)src;
    if (kind == 0)
        hipLaunchKernelGGL(k_mfma_rate<DT_F16>, dim3(blocks), dim3(kThreads), 0, st, s,
                           (float*)out, (unsigned long long*)ticks, steps);
    else if (kind == 1)
        hipLaunchKernelGGL(k_mfma_rate<DT_F8E4M3>, dim3(blocks), dim3(kThreads), 0, st, s,
                           (float*)out, (unsigned long long*)ticks, steps);
    else if (kind == 2)
        hipLaunchKernelGGL(k_mfma_rate<DT_MX_E2M1>, dim3(blocks), dim3(kThreads), 0, st, s,
                           (float*)out, (unsigned long long*)ticks, steps);
    else if (kind == 3)
        hipLaunchKernelGGL(k_mfma_rate<DT_MX_E4M3>, dim3(blocks), dim3(kThreads), 0, st, s,
                           (float*)out, (unsigned long long*)ticks, steps);
    else if (kind == 4)
        hipLaunchKernelGGL(k_smfmac_rate, dim3(blocks), dim3(kThreads), 0, st, s, (float*)out,
                           (unsigned long long*)ticks, steps);
    else
        (void)launch_mfma16_rate(s, (float*)out, (unsigned long long*)ticks, blocks, steps, st);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
