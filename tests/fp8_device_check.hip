// Test support (not part of libmoedx.so): checks on the device that gfx950's
// fp32 -> E4M3FN pack conversion, as the FP8 pack kernel calls it, gives the
// same code as e4m3_code (csrc/fp8_codec.h, itself pinned on the host against
// the oracle's encoder) for every fp32 value of magnitude up to a bound, both
// signs and both halves of the packed word.  The FP8 pack feeds the
// conversion only such finite quotients.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8_codec.h"

namespace {

__global__ void cvt_check_kernel(uint32_t n, uint32_t* __restrict__ mismatches,
                                 uint32_t* __restrict__ first) {
    const uint32_t stride = gridDim.x * blockDim.x;
    uint32_t bad = 0, lowest = 0xffffffffu;
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float q = moedx::fp8_float(i);
        const float nq = moedx::fp8_float(i | 0x80000000u);
        // both word halves, as the pack fills one 32-bit word from 4 quotients
        uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q, nq, 0, false);
        w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(nq, q, (int)w, true);
        const uint32_t cp = moedx::e4m3_code(q), cn = moedx::e4m3_code(nq);
        const uint32_t want = cp | (cn << 8) | (cn << 16) | (cp << 24);
        if (w != want) {
            ++bad;
            lowest = i < lowest ? i : lowest;
        }
    }
    if (bad) {
        atomicAdd(mismatches, bad);
        atomicMin(first, lowest);
    }
}

}  // namespace

// Runs the check over bit patterns [0, n) (and their negatives); returns 0 and
// the mismatch count and lowest mismatching pattern (0xffffffff if none), or a
// HIP error code.
extern "C" __attribute__((visibility("default"))) int fp8_cvt_check(uint32_t n, uint32_t* mismatches,
                                                                   uint32_t* first) {
    uint32_t* d = nullptr;
    hipError_t e = hipMalloc(&d, 8);
    const uint32_t init[2] = {0u, 0xffffffffu};
    if (e == hipSuccess) e = hipMemcpy(d, init, 8, hipMemcpyHostToDevice);
    if (e == hipSuccess) {
        hipLaunchKernelGGL(cvt_check_kernel, dim3(4096), dim3(256), 0, 0, n, d, d + 1);
        e = hipGetLastError();
    }
    uint32_t out[2] = {0u, 0u};
    if (e == hipSuccess) e = hipMemcpy(out, d, 8, hipMemcpyDeviceToHost);
    if (d) (void)hipFree(d);
    *mismatches = out[0];
    *first = out[1];
    return (int)e;
}
