// Measurement helper (not part of the attention path): the shader clock the GPU sustains while
// its matrix cores are busy.  Roofline fractions are quoted against the nominal 2.4 GHz peak
// and, with this figure, against the clock the chip actually ran at.
//
// Every CU runs one workgroup of 4 waves; each wave issues back-to-back bf16 MFMAs on four
// independent accumulators.  Wave 0 of workgroup 0 reads the shader-clock counter (s_memtime)
// and the constant 100 MHz real-time counter (s_memrealtime) before and after its loop; their
// ratio is the clock in MHz.
#include <hip/hip_runtime.h>

#include "hdp_attn.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256, 1) void clock_probe_kernel(int iters, long long* out) {
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(1e-3f * (float)(threadIdx.x + i));
        b[i] = (__bf16)(1e-3f * (float)(i + 1));
    }
    f32x16 acc[4] = {};
    const long long c0 = (long long)__builtin_amdgcn_s_memtime();
    const long long r0 = (long long)__builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    // the loop's results feed a comparison so the MFMAs stay; the store never happens for
    // finite inputs
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    const long long c1 = (long long)__builtin_amdgcn_s_memtime();
    const long long r1 = (long long)__builtin_amdgcn_s_memrealtime();
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        out[0] = c1 - c0;
        out[1] = r1 - r0;
    }
    if (s != s) out[2] = 1;
}

}  // namespace

extern "C" int hdp_probe_clock(int32_t iters, double* mhz, hipStream_t stream) {
    if (iters <= 0 || mhz == nullptr) return HDP_ERR_INVALID_ARG;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return HDP_ERR_HIP;
    long long* d = nullptr;
    long long h[3] = {0, 0, 0};
    if (hipMallocAsync((void**)&d, sizeof(h), stream) != hipSuccess) return HDP_ERR_HIP;
    int rc = HDP_OK;
    if (hipMemcpyAsync(d, h, sizeof(h), hipMemcpyHostToDevice, stream) != hipSuccess) rc = HDP_ERR_HIP;
    if (rc == HDP_OK) {
        hipLaunchKernelGGL(clock_probe_kernel, dim3(cus), dim3(256), 0, stream, iters, d);
        if (hipGetLastError() != hipSuccess) rc = HDP_ERR_HIP;
    }
    if (rc == HDP_OK && (hipMemcpyAsync(h, d, sizeof(h), hipMemcpyDeviceToHost, stream) != hipSuccess ||
                         hipStreamSynchronize(stream) != hipSuccess))
        rc = HDP_ERR_HIP;
    (void)hipFreeAsync(d, stream);
    if (rc != HDP_OK) return rc;
    if (h[1] <= 0) return HDP_ERR_HIP;
    *mhz = (double)h[0] / ((double)h[1] / 100.0);   // cycles per microsecond
    return HDP_OK;
}
