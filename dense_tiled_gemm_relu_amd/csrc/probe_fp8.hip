// Test-only probes of the gfx950 8-bit data paths, with raw per-lane I/O so
// that the host can check the lane layouts the kernel assumes, through the
// kernel's own helpers (InTraits<>::mfma, lds_read_tr8, dma16):
//   * probe_mfma_f8_raw — one v_mfma_f32_32x32x64_f8f6f4 (no block scales):
//     lane l supplies 32 bytes of each operand and returns its 16 results;
//   * probe_tr8_raw — one ds_read_b64_tr_b8 per lane at caller-chosen LDS
//     byte offsets;
//   * probe_unaligned8 — a 16-byte direct global->LDS copy and a 16-byte
//     vector load from any byte offset.
// Built into the probe library only.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gemm_relu_kernel.hpp"

using namespace gemm_relu_hip;

namespace {

// a, b: 64 x 32 bytes (lane-major); d: 64 x 16 floats (lane-major).
// IN_DT: both operands E4M3 or both E5M2.
template <int IN_DT>
__global__ void k_mfma_f8_raw(const uint8_t* a, const uint8_t* b, float* d)
{
    const int l = threadIdx.x;
    i32x8_t av, bv;
    __builtin_memcpy(&av, a + 32 * l, 32);
    __builtin_memcpy(&bv, b + 32 * l, 32);
    f32x16_t acc;
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    acc = InTraits<IN_DT>::mfma(av, bv, acc);
    for (int r = 0; r < 16; ++r) d[16 * l + r] = acc[r];
}

// src: 4096 bytes copied to LDS; lane l reads 8 bytes (transposed) at byte
// offset off[l] (masked to 8-byte alignment inside the buffer); out[8 l + e].
__global__ void k_tr8_raw(const uint8_t* src, const uint32_t* off, uint8_t* out)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[4096];
    for (int i = threadIdx.x; i < 4096; i += 64) lds[i] = src[i];
    __syncthreads();
    const uint32_t o = off[threadIdx.x] & 0xFF8u;
    const i32x2_t v = lds_read_tr8((const GR_LDS unsigned char*)lds + o);
    __builtin_memcpy(out + 8 * threadIdx.x, &v, 8);
}

// Lane l copies 16 bytes starting at byte off[l] of src (any alignment,
// off[l] + 16 <= n, else 0) into LDS with one direct copy, and loads the same
// 16 bytes with a plain vector load: out[0..1023] direct, out[1024..2047] load.
__global__ void k_unaligned8(const uint8_t* src, const uint32_t* off, uint32_t n, uint8_t* out)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[1024];
    for (int i = threadIdx.x; i < 1024; i += 64) lds[i] = 0xFF;
    __syncthreads();
    uint32_t o = off[threadIdx.x];
    if (o + 16 > n) o = 0;   // keep every access inside src
    const GR_LDS unsigned char* base = (const GR_LDS unsigned char*)lds;
    dma16(src, o, lds_addr(base));
    u32x4_t v;
    __builtin_memcpy(&v, src + o, 16);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    for (int i = threadIdx.x; i < 1024; i += 64) out[i] = lds[i];
    __builtin_memcpy(out + 1024 + 16 * threadIdx.x, &v, 16);
}

int finish(hipError_t e)
{
    if (e != hipSuccess) return -3;
    return hipDeviceSynchronize() == hipSuccess ? 0 : -3;
}

}  // namespace

extern "C" int probe_mfma_f8_raw(const void* a, const void* b, void* d, int fmt)
{
    if (fmt == 0)
        k_mfma_f8_raw<DT_F8E4M3><<<1, 64>>>((const uint8_t*)a, (const uint8_t*)b, (float*)d);
    else if (fmt == 1)
        k_mfma_f8_raw<DT_F8E5M2><<<1, 64>>>((const uint8_t*)a, (const uint8_t*)b, (float*)d);
    else
        return -1;
    return finish(hipGetLastError());
}

extern "C" int probe_tr8_raw(const void* src, const void* off, void* out)
{
    k_tr8_raw<<<1, 64>>>((const uint8_t*)src, (const uint32_t*)off, (uint8_t*)out);
    return finish(hipGetLastError());
}

extern "C" int probe_unaligned8(const void* src, const void* off, unsigned n, void* out)
{
    k_unaligned8<<<1, 64>>>((const uint8_t*)src, (const uint32_t*)off, n, (uint8_t*)out);
    return finish(hipGetLastError());
}

// ---- block-scaled (MX) form: v_mfma_scale_f32_32x32x64_f8f6f4 with per-lane
// E8M0 scales.  a, b: 64 x 32 bytes; sa, sb: 64 scale words (byte 0 used);
// d: 64 x 16 floats.  fmt 0: both E4M3; 4: both FP4 E2M1.
namespace {
template <int FMT>
__global__ void k_mfma_mx_raw(const uint8_t* a, const uint8_t* b, const uint32_t* sa,
                              const uint32_t* sb, float* d)
{
    const int l = threadIdx.x;
    i32x8_t av, bv;
    __builtin_memcpy(&av, a + 32 * l, 32);
    __builtin_memcpy(&bv, b + 32 * l, 32);
    f32x16_t acc;
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, FMT, FMT, 0, (int)sa[l], 0,
                                                          (int)sb[l]);
    for (int r = 0; r < 16; ++r) d[16 * l + r] = acc[r];
}
}  // namespace

extern "C" int probe_mfma_mx_raw(const void* a, const void* b, const void* sa, const void* sb,
                                 void* d, int fmt)
{
    if (fmt == 0)
        k_mfma_mx_raw<0><<<1, 64>>>((const uint8_t*)a, (const uint8_t*)b, (const uint32_t*)sa,
                                    (const uint32_t*)sb, (float*)d);
    else if (fmt == 4)
        k_mfma_mx_raw<4><<<1, 64>>>((const uint8_t*)a, (const uint8_t*)b, (const uint32_t*)sa,
                                    (const uint32_t*)sb, (float*)d);
    else
        return -1;
    return finish(hipGetLastError());
}
