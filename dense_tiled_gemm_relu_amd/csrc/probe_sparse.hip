// Test-only probe of the gfx950 2:4 sparse matrix instruction with raw
// per-lane I/O, so that the host can check the operand, index and result
// layouts the sparse kernel assumes:
//   * probe_smfmac_raw — one v_smfmac_f32_32x32x32_{f16,bf16}: lane l supplies
//     8 16-bit values of the compressed (sparse) operand, 16 16-bit values of
//     the dense operand and one 32-bit index word, and returns its 16 results.
// Built into the probe library only.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gemm_relu_kernel.hpp"

using namespace gemm_relu_hip;

namespace {

typedef _Float16 f16x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x16_t __attribute__((ext_vector_type(16)));

// a: 64 x 16 bytes, b: 64 x 32 bytes, idx: 64 words (all lane-major);
// d: 64 x 16 floats.  ABID picks which 16-bit half of the index word is used.
template <bool BF16, int ABID>
__global__ void k_smfmac_raw(const uint8_t* a, const uint8_t* b, const int* idx, float* d)
{
    const int l = threadIdx.x;
    f32x16_t acc;
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    if constexpr (BF16) {
        bf16x8_t av;
        bf16x16_t bv;
        __builtin_memcpy(&av, a + 16 * l, 16);
        __builtin_memcpy(&bv, b + 32 * l, 32);
        acc = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(av, bv, acc, idx[l], 0, ABID);
    } else {
        f16x8_t av;
        f16x16_t bv;
        __builtin_memcpy(&av, a + 16 * l, 16);
        __builtin_memcpy(&bv, b + 32 * l, 32);
        acc = __builtin_amdgcn_smfmac_f32_32x32x32_f16(av, bv, acc, idx[l], 0, ABID);
    }
    for (int r = 0; r < 16; ++r) d[16 * l + r] = acc[r];
}

int finish(hipError_t e)
{
    if (e != hipSuccess) return -2;
    return hipDeviceSynchronize() == hipSuccess ? 0 : -3;
}

}  // namespace

// dtype 0: f16, 1: bf16; abid 0 or 1.  Returns 0, or -1 for a bad argument,
// -2 / -3 for a launch / execution failure.
extern "C" int probe_smfmac_raw(const void* a, const void* b, const void* idx, void* d, int dtype,
                                int abid)
{
    const uint8_t* pa = (const uint8_t*)a;
    const uint8_t* pb = (const uint8_t*)b;
    const int* pi = (const int*)idx;
    float* pd = (float*)d;
    if (dtype == 0 && abid == 0)
        k_smfmac_raw<false, 0><<<1, 64>>>(pa, pb, pi, pd);
    else if (dtype == 0 && abid == 1)
        k_smfmac_raw<false, 1><<<1, 64>>>(pa, pb, pi, pd);
    else if (dtype == 1 && abid == 0)
        k_smfmac_raw<true, 0><<<1, 64>>>(pa, pb, pi, pd);
    else if (dtype == 1 && abid == 1)
        k_smfmac_raw<true, 1><<<1, 64>>>(pa, pb, pi, pd);
    else
        return -1;
    return finish(hipGetLastError());
}
