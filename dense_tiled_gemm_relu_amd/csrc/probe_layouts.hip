// Test-only probes of the gfx950 data movements the GEMM kernel relies on.
// Each runs one wave (64 threads) on tiny in-bounds buffers and reports what
// the hardware did, through the same helpers the kernel uses:
//   * probe_mfma_32x32x16, probe_mfma_16x16x32 — one MFMA with the operand /
//     result lane layouts the kernel assumes; the host compares D with X·Y;
//   * probe_tr16 — one transpose read per lane at caller-chosen LDS offsets;
//   * probe_dma16 — one 16-byte direct global->LDS copy per lane.
// Built into its own library; the product library does not contain these.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gemm_relu_kernel.hpp"

using namespace gemm_relu_hip;

namespace {

// X: 32 x 16 row-major, Y: 16 x 32 row-major (16-bit patterns), D: 32 x 32 fp32.
// Lane l feeds X[l % 32][8 (l / 32) + e] and Y[8 (l / 32) + e][l % 32], e = 0..7,
// and owns D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32] in result register r.
template <int IN_DT>
__global__ void k_mfma(const uint16_t* X, const uint16_t* Y, float* D)
{
    const int l = threadIdx.x, r32 = l & 31, g = l >> 5;
    i16x8_t a, b;
    for (int e = 0; e < 8; ++e) {
        a[e] = (short)X[r32 * 16 + 8 * g + e];
        b[e] = (short)Y[(8 * g + e) * 32 + r32];
    }
    f32x16_t acc;
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    acc = InTraits<IN_DT>::mfma(a, b, acc);
    for (int r = 0; r < 16; ++r) D[(8 * (r / 4) + 4 * g + r % 4) * 32 + r32] = acc[r];
}

// src: 4096 16-bit values copied to LDS; lane l reads 8 bytes (transposed) at
// byte offset off[l] (must be < 8192 - 8 and 8-byte aligned); out[4 l + e].
__global__ void k_tr16(const uint16_t* src, const uint32_t* off, uint16_t* out)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds[4096];
    for (int i = threadIdx.x; i < 4096; i += 64) lds[i] = src[i];
    __syncthreads();
    const GR_LDS unsigned char* base = (const GR_LDS unsigned char*)lds;
    const i16x4_t v = lds_read_tr16(base + (off[threadIdx.x] & 0x1FF8u));   // in bounds, 8-byte aligned
    for (int e = 0; e < 4; ++e) out[4 * threadIdx.x + e] = (uint16_t)v[e];
}

// Lane l copies the 16-byte chunk chunk[l] (< 64) of src into LDS with one
// direct copy; the LDS contents (64 x 16 bytes) are then written to out.
__global__ void k_dma16(const uint16_t* src, const uint32_t* chunk, uint16_t* out)
{
    __shared__ __attribute__((aligned(1024))) uint16_t lds[512];
    for (int i = threadIdx.x; i < 512; i += 64) lds[i] = 0xFFFF;
    __syncthreads();
    const GR_LDS unsigned char* base = (const GR_LDS unsigned char*)lds;
    dma16(reinterpret_cast<const unsigned char*>(src), (chunk[threadIdx.x] & 63u) * 16u, lds_addr(base));
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    for (int i = threadIdx.x; i < 512; i += 64) out[i] = lds[i];
}

// Lane l copies 16 bytes starting at element off[l] of src (2-byte aligned,
// in bounds: off[l] + 8 <= n) into LDS with one direct copy, and also loads the
// same 16 bytes into registers with a plain vector load; both land in out
// (direct copy: out[0..511], register load: out[512..1023]).
__global__ void k_unaligned16(const uint16_t* src, const uint32_t* off, uint32_t n, uint16_t* out)
{
    __shared__ __attribute__((aligned(1024))) uint16_t lds[512];
    for (int i = threadIdx.x; i < 512; i += 64) lds[i] = 0xFFFF;
    __syncthreads();
    uint32_t o = off[threadIdx.x];
    if (o + 8 > n) o = 0;   // keep every access inside src
    const GR_LDS unsigned char* base = (const GR_LDS unsigned char*)lds;
    dma16(reinterpret_cast<const unsigned char*>(src), o * 2u, lds_addr(base));
    u32x4_t v;
    __builtin_memcpy(&v, src + o, 16);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    for (int i = threadIdx.x; i < 512; i += 64) out[i] = lds[i];
    *reinterpret_cast<u32x4_t*>(out + 512 + 8 * threadIdx.x) = v;
}

// X: 16 x 32 row-major, Y: 32 x 16 row-major (16-bit patterns), D: 16 x 16 fp32.
// Lane l feeds X[l % 16][8 (l / 16) + e] and Y[8 (l / 16) + e][l % 16], e = 0..7,
// and owns D[4 (l / 16) + r][l % 16] in result register r.
template <int IN_DT>
__global__ void k_mfma16(const uint16_t* X, const uint16_t* Y, float* D)
{
    const int l = threadIdx.x, r16 = l & 15, g = l >> 4;
    i16x8_t a, b;
    for (int e = 0; e < 8; ++e) {
        a[e] = (short)X[r16 * 32 + 8 * g + e];
        b[e] = (short)Y[(8 * g + e) * 16 + r16];
    }
    f32x4_t acc;
    for (int r = 0; r < 4; ++r) acc[r] = 0.0f;
    acc = InTraits<IN_DT, 16>::mfma(a, b, acc);
    for (int r = 0; r < 4; ++r) D[(4 * g + r) * 16 + r16] = acc[r];
}

int finish(hipError_t e)
{
    if (e != hipSuccess) return -3;
    return hipDeviceSynchronize() == hipSuccess ? 0 : -3;
}

}  // namespace

extern "C" int probe_mfma_32x32x16(const void* X, const void* Y, void* D, int in_dtype)
{
    if (in_dtype == 0)
        k_mfma<DT_F16><<<1, 64>>>((const uint16_t*)X, (const uint16_t*)Y, (float*)D);
    else
        k_mfma<DT_BF16><<<1, 64>>>((const uint16_t*)X, (const uint16_t*)Y, (float*)D);
    return finish(hipGetLastError());
}

extern "C" int probe_mfma_16x16x32(const void* X, const void* Y, void* D, int in_dtype)
{
    if (in_dtype == 0)
        k_mfma16<DT_F16><<<1, 64>>>((const uint16_t*)X, (const uint16_t*)Y, (float*)D);
    else
        k_mfma16<DT_BF16><<<1, 64>>>((const uint16_t*)X, (const uint16_t*)Y, (float*)D);
    return finish(hipGetLastError());
}

extern "C" int probe_tr16(const void* src, const void* off, void* out)
{
    k_tr16<<<1, 64>>>((const uint16_t*)src, (const uint32_t*)off, (uint16_t*)out);
    return finish(hipGetLastError());
}

extern "C" int probe_unaligned16(const void* src, const void* off, unsigned n, void* out)
{
    k_unaligned16<<<1, 64>>>((const uint16_t*)src, (const uint32_t*)off, n, (uint16_t*)out);
    return finish(hipGetLastError());
}

extern "C" int probe_dma16(const void* src, const void* chunk, void* out)
{
    k_dma16<<<1, 64>>>((const uint16_t*)src, (const uint32_t*)chunk, (uint16_t*)out);
    return finish(hipGetLastError());
}
